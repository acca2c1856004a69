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
// both with the model dimension contiguous.  Block: 256 features x 256
// tokens; 8 wavefronts, each 64 features x 128 tokens (4 x 8 tiles of
// v_mfma_f32_16x16x32_bf16), so every operand read from LDS feeds 4 or 8
// MFMAs.  The model dimension is walked in 32-wide steps through five LDS
// stages (5 x 32 KB): the tiles move from global memory straight into LDS
// (global_load_lds_dwordx4, no staging registers, no LDS store instructions)
// four steps ahead of their use, spread among the MFMAs, and the operands of
// step st + 1 are read from LDS while the MFMAs of step st run.
#include <type_traits>

#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

constexpr int kPF = 256;        // features per block
constexpr int kPT = 256;        // tokens per block
constexpr int kPK = 32;         // model-dimension step
constexpr int kPStages = 5;     // LDS stages (loads run kPStages - 1 steps ahead)
constexpr int kPWaves = 8;
constexpr int kXcdsP = 8;
constexpr int kGroupT = 8;      // token blocks per L2 group

// One 16-byte direct global-to-LDS load per lane (global_load_lds_dwordx4,
// scalar-base form): lane i reads base + voff_bytes and writes LDS bytes
// lds + 16 i .. lds + 16 i + 15; base and lds are wavefront-uniform (SGPRs,
// lds through M0).  Written as assembly so that the compiler does not track
// it: its own bookkeeping of such loads turns conservative with several LDS
// stages in flight and makes every LDS read wait for all of them.  The kernel
// orders its LDS reads after these loads itself (wait_stage), and leaves M0
// to them alone.  An LDS DMA reads M0 one wait state after the scalar write
// at the earliest, hence the s_nop.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff_bytes, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff_bytes),
                 "s"(base)
                 : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}
// f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
// Sixteen bytes from LDS through an explicit LDS pointer.
__device__ __forceinline__ u32x4 lds_read16(const uint16_t *p) {
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    return *(lds_u32x4 *)(p);
}
// All but this thread's N most recent direct loads have landed (they
// complete in order), then a workgroup barrier that itself waits for nothing.
template <int N>
__device__ __forceinline__ void wait_stage() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 7 and lgkmcnt 15 (no wait).
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// 16-byte chunk c (0..3) of LDS row r (32 elements, 64 bytes, no padding)
// sits at chunk c ^ swz(r).  An operand read has lane group grp read chunk
// grp of 16 consecutive rows.  Measured on gfx950 (ds_read_b128, 8
// wavefronts per CU): with swz(r) = (r >> 1) & 3 these reads take the 32
// cycles per instruction that contiguous reads take; with (r >> 2) & 3 they
// take 58, and unswizzled 64-byte rows 58 as well.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

__global__ __launch_bounds__(kPWaves *kWave, 2) void projection_kernel(ProjectionParams p) {
    using S = uint16_t;
    // Five stages of the weight and token tiles (a stage: 256 weight rows,
    // then 256 token rows, 32 elements each; 160 KB in all), carved from one
    // array that afterwards holds the block's output tile.
    constexpr int kStage = (kPF + kPT) * kPK;
    __shared__ __attribute__((aligned(16))) S lds[kPStages * kStage];
    static_assert(kPStages * kStage >= kPF * kPT, "the output tile reuses the stages");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int wf = wave & 3, wt = wave >> 2;

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

    // Direct loads: slot n of this thread is LDS chunk (n * 8 + wave) * 64 + lane
    // of the tile: row slot / CPR, physical chunk slot % CPR, holding global
    // chunk (physical ^ swz(row)) of that row.  Rows past the end of the
    // weight or of the tokens re-read the last row (their results are not
    // stored).  Byte offsets are taken from the block's first row, so they
    // stay below 2^32 for any d_model up to 2^22.
    constexpr int CPR = kPK / 8;
    constexpr int NDW = kPF * CPR / (kPWaves * kWave);
    constexpr int NDX = kPT * CPR / (kPWaves * kWave);
    static_assert(NDW * kPWaves * kWave == kPF * CPR && NDX * kPWaves * kWave == kPT * CPR, "loader shape");
    const S *wblk = wg + static_cast<int64_t>(f0) * K;
    const S *xblk = xg + static_cast<int64_t>(t0) * K;
    uint32_t wsrc[NDW], xsrc[NDX];
#pragma unroll
    for (int n = 0; n < NDW; ++n) {
        const int s = (n * kPWaves + wave) * kWave + lane, r = s / CPR, c = (s % CPR) ^ swz(r);
        wsrc[n] = static_cast<uint32_t>((static_cast<int64_t>(min(f0 + r, n_feat - 1) - f0) * K + c * 8) * 2);
    }
#pragma unroll
    for (int n = 0; n < NDX; ++n) {
        const int s = (n * kPWaves + wave) * kWave + lane, r = s / CPR, c = (s % CPR) ^ swz(r);
        xsrc[n] = static_cast<uint32_t>((min(static_cast<int64_t>(t0 + r), M - 1) - t0) * K * 2 + c * 16);
    }
    const int n_steps = K / kPK;
    const uint32_t wave_off = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave) * kWave * 16);
    // Load n (0 .. NDW + NDX - 1) of step st (clamped to the last step: the
    // loads past the end are harmless reloads that keep the number in flight
    // constant) into the stage at lw.
    auto dma_one = [&](int n, int st, const S *lw) __attribute__((always_inline)) {
        const uint32_t kb = static_cast<uint32_t>(min(st, n_steps - 1) * kPK * 2);
        if (n < NDW) dma16(wblk, wsrc[n] + kb, lds_address(lw) + wave_off + n * kPWaves * kWave * 16);
        else dma16(xblk, xsrc[n - NDW] + kb, lds_address(lw + kPF * kPK) + wave_off + (n - NDW) * kPWaves * kWave * 16);
    };
    constexpr int ND = NDW + NDX;

    constexpr int NI = 4, NJ = 8;
    static_assert(ND <= NI, "one load per row of MFMAs");
    f32x4 acc[NI][NJ];
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int b = 0; b < NJ; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Lane read offsets: row 16 i + col of the wavefront's part, chunk grp,
    // swizzled by swz(row) = swz(col) (the part starts on a multiple of 16
    // rows, and swz depends on row bits 1-2 only).
    const int aoff = (16 * NI * wf + col) * kPK + (grp ^ swz(col)) * 8;
    const int boff = (16 * NJ * wt + col) * kPK + (grp ^ swz(col)) * 8;
    struct Ops {
        Op8<BF16> a[NI], b[NJ];
    };
    auto read_ops = [&](Ops &o, int stage) __attribute__((always_inline)) {
        const S *tw = lds + stage * kStage, *tx = tw + kPF * kPK;
#pragma unroll
        for (int i = 0; i < NI; ++i) o.a[i].w = lds_read16(tw + aoff + 16 * i * kPK);
#pragma unroll
        for (int j = 0; j < NJ; ++j) o.b[j].w = lds_read16(tx + boff + 16 * j * kPK);
    };
    // Step st: read the operands of step st + 1 (its stage landed before the
    // last barrier), then the MFMAs of step st with the loads of step st + 4
    // into the stage step st - 1 read spread among them -- the CU's memory
    // pipeline takes these 1 KB requests at about 64 bytes a clock, so a
    // wavefront issuing them back to back would stall -- then wait until only
    // the loads of steps st + 3 and st + 4 are outstanding, i.e. step st + 2
    // has landed for every thread, and meet at the barrier.
    Ops ops0, ops1;
    auto step = [&](int st, auto u_c, Ops &cur, Ops &nxt) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;
        if (st + 1 < n_steps) read_ops(nxt, (U + 1) % kPStages);
        const S *lw = lds + ((U + kPStages - 1) % kPStages) * kStage;
        static_for<0, NI>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int I = decltype(i_c)::value;
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[I][j] = mma32(cur.a[I], cur.b[j], acc[I][j]);
            if constexpr (I < ND) {
                __builtin_amdgcn_sched_barrier(0);
                dma_one(I, st + kPStages - 1, lw);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        wait_stage<(kPStages - 3) * ND>();
    };

    for (int st = 0; st < kPStages - 1; ++st)
#pragma unroll
        for (int n = 0; n < ND; ++n) dma_one(n, st, lds + st * kStage);
    wait_stage<(kPStages - 3) * ND>();  // steps 0 and 1 have landed
    read_ops(ops0, 0);
    // Unrolled by ten so that every stage (st % 5) and operand set (st % 2)
    // is named statically.
    for (int st = 0; st < n_steps; st += 2 * kPStages) {
        static_for<0, 2 * kPStages>([&](auto u) __attribute__((always_inline)) {
            constexpr int U = decltype(u)::value;
            if (st + U < n_steps) {
                if constexpr (U % 2 == 0) step(st + U, std::integral_constant<int, U % kPStages>{}, ops0, ops1);
                else step(st + U, std::integral_constant<int, U % kPStages>{}, ops1, ops0);
            }
        });
    }
    // The reloads past the end are still in flight: they land before the
    // stages are overwritten with the output tile.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Epilogue through LDS: the stages are free once every wavefront has read
    // its last one, and the 256 x 256 output tile (bf16, 128 KB) goes there
    // as [token][feature] rows of 512 bytes; then each 16-byte chunk of a
    // row -- 8 consecutive features, never across a head or a tensor, since
    // d and the q/k/v/probe boundaries are multiples of 8 -- is stored with
    // one 16-byte write, so the 16 chunks of a (token, head) row of d = 128
    // go out as one 256-byte run.
    // Row r keeps its 16-byte chunk c at c ^ (r % 16): the 16 tokens (rows
    // r % 16 = col) of one accumulator write then spread over the banks, and
    // a chunk's two 8-byte halves stay adjacent.
    constexpr int ORS = kPF;  // output tile row: 256 features
    {
        // acc[i][j][e] is feature 128 wf + 16 i + 4 grp + e of token
        // 128 wt + 16 j + col of the block.
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            S *row = lds + (16 * NJ * wt + 16 * j + col) * ORS;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int u = 4 * NI * wf + 4 * i + grp;  // 8-byte unit within the row
                const float y[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                store4(row + 4 * (u ^ (2 * col)), y);
            }
        }
    }
    __syncthreads();
    // Thread tid stores chunk tid % 32 (features 8 (tid % 32) ..) of rows
    // RPI it + tid / 32, it = 0 .. kPT / RPI - 1.
    constexpr int RPI = kPWaves * kWave / 32;  // rows per pass
    const int c16 = tid & 31;
    const int f = f0 + 8 * c16;
    if (f < n_feat) {
        S *base;
        int H, fl;
        if (f < p.nq) {
            base = static_cast<S *>(p.q); H = p.Hq; fl = f;
        } else if (f < p.nq + p.nkv) {
            base = static_cast<S *>(p.k); H = p.Hkv; fl = f - p.nq;
        } else if (f < p.nq + 2 * p.nkv) {
            base = static_cast<S *>(p.v); H = p.Hkv; fl = f - p.nq - p.nkv;
        } else {
            base = static_cast<S *>(p.rho); H = p.Hq; fl = f - p.nq - 2 * p.nkv;
        }
        const int h = fl / p.d, a = fl % p.d;
#pragma unroll
        for (int it = 0; it < kPT / RPI; ++it) {
            const int r = RPI * it + (tid >> 5);
            const int64_t t = t0 + r;
            if (t >= M) break;
            const u32x4 val = lds_read16(lds + r * ORS + 8 * (c16 ^ (r & 15)));
            const int64_t bb = t / p.T, tt = t - bb * p.T;
            *reinterpret_cast<u32x4 *>(base + ((bb * H + h) * p.T + tt) * p.d + a) = val;
        }
    }
}

}  // namespace

int projection_block_features() { return kPF; }
int projection_block_tokens() { return kPT; }
// d_model granularity the entry point accepts (the kernel needs kPK).
int projection_step() { return 2 * kPK; }

hipError_t launch_projection(const ProjectionParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(projection_kernel, dim3(static_cast<uint32_t>(p.n_fblk) * p.n_tblk), dim3(kPWaves * kWave),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace plx
