// plx_diag.hip -- measurement aids: device facts from the HIP runtime, a
// plain streaming-read kernel and a bf16 matrix-core throughput kernel.  They
// measure the ceilings that the attention kernels are read against and share
// nothing with those kernels.
#include <stdint.h>

#include "../../include/parallax_diag.h"
#include "plx_device.h"

namespace plx {

namespace {

constexpr int kDiagThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread
constexpr uint32_t kSinkX = 0x9e3779b9u, kSinkY = 0x7f4a7c15u;

template <bool NT>
__global__ __launch_bounds__(kDiagThreads) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n_vec,
                                                                  uint32_t *sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kDiagThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kDiagThreads + threadIdx.x;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (; i + (kReadUnroll - 1) * stride < n_vec; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    for (; i < n_vec; i += stride) acc ^= NT ? __builtin_nontemporal_load(src + i) : src[i];
    if (acc.x == kSinkX && acc.y == kSinkY) sink[0] = acc.z;
}

// Each wavefront: iterations x 8 MFMAs on eight independent accumulators, so
// every MFMA can issue as soon as the matrix core is free.  The occupancy
// hint keeps the accumulators in place across iterations: without it the
// register allocator rotates them through copies inside the loop.
__global__ __launch_bounds__(kDiagThreads, 2) void mfma_bf16_kernel(uint32_t *sink, int iterations) {
    const int l = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(0.001f * static_cast<float>(l + e));
        b[e] = static_cast<__bf16>(0.002f * static_cast<float>(l - e));
    }
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iterations; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    f32x4 s = acc[0];
#pragma unroll
    for (int c = 1; c < 8; ++c) s += acc[c];
    const uint32_t x = __float_as_uint(s[0]), y = __float_as_uint(s[1]);
    if (x == kSinkX && y == kSinkY) sink[0] = __float_as_uint(s[2]);
}

}  // namespace

}  // namespace plx

extern "C" {

plx_status_t parallax_diag_device_info(int32_t device, int32_t *cu_count, int32_t *max_clock_khz) {
    if (!cu_count || !max_clock_khz) return PLX_ERR_INVALID_ARGUMENT;
    int cu = 0, clk = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device) != hipSuccess)
        return PLX_ERR_HIP;
    *cu_count = cu;
    *max_clock_khz = clk;
    return PLX_OK;
}

plx_status_t parallax_diag_stream_read(const void *src, size_t bytes, int32_t nontemporal, void *sink,
                                       hipStream_t stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0) return PLX_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return PLX_ERR_INVALID_ARGUMENT;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), k0 = reinterpret_cast<uintptr_t>(sink);
    if (k0 < s0 + bytes && s0 < k0 + 4) return PLX_ERR_INVALID_ARGUMENT;
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PLX_ERR_HIP;
    const int64_t n_vec = static_cast<int64_t>(bytes / 16);
    int64_t blocks = 2 * static_cast<int64_t>(cu > 0 ? cu : 1);
    const int64_t need = (n_vec + plx::kDiagThreads - 1) / plx::kDiagThreads;
    if (blocks > need) blocks = need;
    const auto *p = static_cast<const plx::u32x4 *>(src);
    auto *out = static_cast<uint32_t *>(sink);
    auto st = stream;
    if (nontemporal)
        hipLaunchKernelGGL(plx::stream_read_kernel<true>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(plx::kDiagThreads), 0, st, p, n_vec, out);
    else
        hipLaunchKernelGGL(plx::stream_read_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(plx::kDiagThreads), 0, st, p, n_vec, out);
    return hipGetLastError() == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t parallax_diag_mfma_bf16(void *sink, int32_t n_blocks, int32_t iterations, hipStream_t stream) {
    if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return PLX_ERR_INVALID_ARGUMENT;
    if (n_blocks < 1 || n_blocks > (1 << 20) || iterations < 1 || iterations > (1 << 24))
        return PLX_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(plx::mfma_bf16_kernel, dim3(static_cast<uint32_t>(n_blocks)), dim3(plx::kDiagThreads), 0,
                       stream, static_cast<uint32_t *>(sink), iterations);
    return hipGetLastError() == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

}  // extern "C"
