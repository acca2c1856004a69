// plx_projection.hip -- fused q/k/v/probe projection on gfx950 (bf16 in and
// out, fp32 accumulation).
//
// The probe is a learned linear map of the layer input, rho = W_R x (the
// news.chathome.org article on Parallax, "What is Parallax"; the gist.science
// summary, "Method: Parallax / core mechanism").  It is computed here as one
// more block of output features of the q/k/v projection: one GEMM over the
// stacked weight [(Hq + Hkv + Hkv + Hq) d, d_model] (torch Linear layout, a
// row per output feature: q heads, k heads, v heads, probe heads), whose
// results are written straight into the attention layout [B, H, T, d], so no
// separate transpose pass exists.
//
// The kernel computes C^T = W x^T: output features along the MFMA rows (A
// operand = weight rows), tokens along the columns (B operand = token rows),
// both with the model dimension contiguous, so each lane ends up holding 4
// consecutive head dimensions of one token and writes them with one 8-byte
// store.  Block: 256 features x 256 tokens, 64-wide steps over d_model,
// double-buffered in LDS (exactly the 160 KB of a CU); 8 wavefronts, each 64
// features x 128 tokens (4 x 8 tiles of v_mfma_f32_16x16x32_bf16), so every
// operand read from LDS feeds 4 or 8 MFMAs.
#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

constexpr int kPF = 256;        // features per block
constexpr int kPT = 256;        // tokens per block
constexpr int kPK = 64;         // model-dimension step
constexpr int kPRS = kPK + 16;  // LDS row stride (elements): 160-byte rows; measured against 144, 176 and 192 bytes, 4% faster
constexpr int kPWaves = 8;
constexpr int kXcdsP = 8;
constexpr int kGroupT = 8;      // token blocks per L2 group

__global__ __launch_bounds__(kPWaves *kWave, 2) void projection_kernel(ProjectionParams p) {
    using S = uint16_t;
    __shared__ __attribute__((aligned(16))) S lds_w[2][kPF * kPRS];
    __shared__ __attribute__((aligned(16))) S lds_x[2][kPT * kPRS];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int wf = wave & 3, wt = wave >> 2;  // wavefront's 64-feature x 128-token tile of the block

    // Block order: workgroups are dealt to the 8 XCDs round-robin.  Within an
    // XCD, blocks run in groups of kGroupT token blocks, feature block outer,
    // so the blocks in flight on one XCD share a few weight and token slabs.
    int fblk, tblk;
    {
        const int id = blockIdx.x;
        int slot = id, xcd = 0, per = p.n_tblk;
        if (p.n_tblk % kXcdsP == 0) {
            xcd = id % kXcdsP;
            slot = id / kXcdsP;
            per = p.n_tblk / kXcdsP;
        }
        const int span = kGroupT * p.n_fblk;
        const int group = slot / span, in = slot % span;
        const int gsize = min(kGroupT, per - group * kGroupT);
        fblk = in / gsize;
        const int tloc = group * kGroupT + in % gsize;
        tblk = p.n_tblk % kXcdsP == 0 ? xcd + kXcdsP * tloc : tloc;
    }
    const int f0 = fblk * kPF;
    const int t0 = tblk * kPT;
    const int K = p.d_model;
    const int64_t M = p.n_tokens;

    const int n_feat = p.nq * 2 + p.nkv * 2;
    const S *wg = static_cast<const S *>(p.w);
    const S *xg = static_cast<const S *>(p.x);

    // Loaders: 16-byte chunks, NWC of the weight tile and NXC of the token
    // tile per thread; rows past the last feature or token are clamped (their
    // results are not stored).
    constexpr int NTHR = kPWaves * kWave;
    constexpr int NWC = kPF * kPK / 8 / NTHR;
    constexpr int NXC = kPT * kPK / 8 / NTHR;
    int wl[NWC], xl[NXC];
    int64_t wrow[NWC], xrow[NXC];
#pragma unroll
    for (int n = 0; n < NWC; ++n) {
        const int c = tid + n * NTHR;
        wl[n] = (c / (kPK / 8)) * kPRS + (c % (kPK / 8)) * 8;
        wrow[n] = static_cast<int64_t>(min(f0 + c / (kPK / 8), n_feat - 1)) * K + (c % (kPK / 8)) * 8;
    }
#pragma unroll
    for (int n = 0; n < NXC; ++n) {
        const int c = tid + n * NTHR;
        xl[n] = (c / (kPK / 8)) * kPRS + (c % (kPK / 8)) * 8;
        xrow[n] = min(static_cast<int64_t>(t0 + c / (kPK / 8)), M - 1) * K + (c % (kPK / 8)) * 8;
    }
    Op8<BF16> sw[NWC], sx[NXC];
    auto load = [&](int kk) {
#pragma unroll
        for (int n = 0; n < NWC; ++n) sw[n] = op8_load(wg + wrow[n] + kk);
#pragma unroll
        for (int n = 0; n < NXC; ++n) sx[n] = op8_load(xg + xrow[n] + kk);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int n = 0; n < NWC; ++n) store_op8(&lds_w[buf][wl[n]], sw[n]);
#pragma unroll
        for (int n = 0; n < NXC; ++n) store_op8(&lds_x[buf][xl[n]], sx[n]);
    };

    constexpr int NI = 4, NJ = 8;  // 16 x 16 tiles per wavefront: features x tokens
    f32x4 acc[NI][NJ];
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int b = 0; b < NJ; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_steps = K / kPK;
    load(0);
    store(0);
    for (int s = 0; s < n_steps; ++s) {
        const int buf = s & 1;
        __syncthreads();
        const bool more = s + 1 < n_steps;
        if (more) load((s + 1) * kPK);
        const S *tw = lds_w[buf] + (16 * NI * wf) * kPRS;
        const S *tx = lds_x[buf] + (16 * NJ * wt) * kPRS;
#pragma unroll
        for (int ks = 0; ks < kPK / 32; ++ks) {
            Op8<BF16> a[NI], b[NJ];
#pragma unroll
            for (int i = 0; i < NI; ++i) a[i] = op8_load(tw + (16 * i + col) * kPRS + 32 * ks + 8 * grp);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = op8_load(tx + (16 * j + col) * kPRS + 32 * ks + 8 * grp);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mma32(a[i], b[j], acc[i][j]);
        }
        if (more) store(buf ^ 1);
    }

    // acc[i][j][e] is feature f0 + 64 wf + 16 i + 4 grp + e of token
    // t0 + 128 wt + 16 j + col.  Four consecutive features share a head.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int64_t t = t0 + 16 * NJ * wt + 16 * j + col;
        if (t >= M) continue;
        const int64_t bb = t / p.T, tt = t % p.T;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            int f = f0 + 16 * NI * wf + 16 * i + 4 * grp;
            if (f >= n_feat) continue;
            void *base;
            int H;
            if (f < p.nq) {
                base = p.q; H = p.Hq;
            } else if (f < p.nq + p.nkv) {
                base = p.k; H = p.Hkv; f -= p.nq;
            } else if (f < p.nq + 2 * p.nkv) {
                base = p.v; H = p.Hkv; f -= p.nq + p.nkv;
            } else {
                base = p.rho; H = p.Hq; f -= p.nq + 2 * p.nkv;
            }
            const int h = f / p.d, a = f % p.d;
            S *dst = static_cast<S *>(base) + ((bb * H + h) * p.T + tt) * p.d + a;
            float y[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            store4(dst, y);
        }
    }
}

}  // namespace

int projection_block_features() { return kPF; }
int projection_block_tokens() { return kPT; }
int projection_step() { return kPK; }

hipError_t launch_projection(const ProjectionParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(projection_kernel, dim3(static_cast<uint32_t>(p.n_fblk) * p.n_tblk), dim3(kPWaves * kWave),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace plx
