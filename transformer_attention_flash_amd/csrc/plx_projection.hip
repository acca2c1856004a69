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
// double-buffered in LDS (128 KB); 8 wavefronts, each 64 features x 128
// tokens (4 x 8 tiles of v_mfma_f32_16x16x32_bf16), so every operand read
// from LDS feeds 4 or 8 MFMAs.  The tiles move from global memory straight
// into LDS (global_load_lds_dwordx4, no staging registers, no LDS store
// instructions): 6% faster than loads staged through registers into padded
// rows.
#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

constexpr int kPF = 256;        // features per block
constexpr int kPT = 256;        // tokens per block
constexpr int kPK = 64;         // model-dimension step
constexpr int kPWaves = 8;
constexpr int kXcdsP = 8;
constexpr int kGroupT = 8;      // token blocks per L2 group

// One 16-byte direct global-to-LDS load per lane (global_load_lds_dwordx4):
// lane i writes bytes 16 i .. 16 i + 15 from the wavefront-uniform LDS
// address `lds`.
__device__ __forceinline__ void lds_load16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
// An offset the optimizer cannot take apart (one move, outside the loop): the
// compiler keeps its LDS alias information only for short address chains.
__device__ __forceinline__ int opaque(int x) { return __builtin_amdgcn_mov_dpp(x, 0xE4, 0xF, 0xF, false); }
// 16-byte chunk c of LDS row r (64 elements, 128 bytes, no padding) sits at
// chunk c ^ swz(r).  Two rows share one 256-byte bank row, so the 16-byte bank
// group of (r, c) is 8 (r & 1) + (c ^ swz(r)): for the 16 lanes that read
// chunk c of 16 consecutive rows these are 16 different groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kPWaves *kWave, 2) void projection_kernel(ProjectionParams p) {
    using S = uint16_t;
    // Two stages of the weight and token tiles, each buffer its own LDS array
    // so that the compiler can tell the direct loads into one stage from the
    // reads of the other.
    __shared__ __attribute__((aligned(16))) S lds_w0[kPF * kPK], lds_w1[kPF * kPK];
    __shared__ __attribute__((aligned(16))) S lds_x0[kPT * kPK], lds_x1[kPT * kPK];

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
    // of the tile: row slot / 8, physical chunk slot % 8, holding global chunk
    // (physical ^ swz(row)) of that row.
    constexpr int CPR = kPK / 8;
    constexpr int NDW = kPF * CPR / (kPWaves * kWave);
    constexpr int NDX = kPT * CPR / (kPWaves * kWave);
    int64_t wsrc[NDW], xsrc[NDX];
#pragma unroll
    for (int n = 0; n < NDW; ++n) {
        const int s = (n * kPWaves + wave) * kWave + lane, r = s / CPR, c = (s % CPR) ^ swz(r);
        wsrc[n] = static_cast<int64_t>(min(f0 + r, n_feat - 1)) * K + c * 8;
    }
#pragma unroll
    for (int n = 0; n < NDX; ++n) {
        const int s = (n * kPWaves + wave) * kWave + lane, r = s / CPR, c = (s % CPR) ^ swz(r);
        xsrc[n] = min(static_cast<int64_t>(t0 + r), M - 1) * K + c * 8;
    }
    auto dma = [&](int kk, S *lw, S *lx) {
#pragma unroll
        for (int n = 0; n < NDW; ++n) lds_load16(wg + wsrc[n] + kk, lw + (n * kPWaves + wave) * kWave * 8);
#pragma unroll
        for (int n = 0; n < NDX; ++n) lds_load16(xg + xsrc[n] + kk, lx + (n * kPWaves + wave) * kWave * 8);
    };

    constexpr int NI = 4, NJ = 8;
    f32x4 acc[NI][NJ];
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int b = 0; b < NJ; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Lane read offsets: row 16 i + col of the wavefront's part, chunk
    // 4 ks + grp, swizzled by swz(row) = swz(col) (the part starts on a
    // multiple of 16 rows).
    int aoff[kPK / 32], boff[kPK / 32];
#pragma unroll
    for (int ks = 0; ks < kPK / 32; ++ks) {
        aoff[ks] = opaque((16 * NI * wf + col) * kPK + ((4 * ks + grp) ^ swz(col)) * 8);
        boff[ks] = opaque((16 * NJ * wt + col) * kPK + ((4 * ks + grp) ^ swz(col)) * 8);
    }
    auto compute = [&](const S *tw, const S *tx) {
#pragma unroll
        for (int ks = 0; ks < kPK / 32; ++ks) {
            Op8<BF16> a[NI], b[NJ];
#pragma unroll
            for (int i = 0; i < NI; ++i) a[i] = op8_load(tw + aoff[ks] + 16 * i * kPK);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = op8_load(tx + boff[ks] + 16 * j * kPK);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mma32(a[i], b[j], acc[i][j]);
        }
    };

    const int n_steps = K / kPK;
    dma(0, lds_w0, lds_x0);
    for (int s = 0; s < n_steps; s += 2) {
        // Stage s is in buffer 0, stage s + 1 goes to buffer 1 (free: its last
        // readers finished stage s - 1 before this barrier), and so on.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's direct loads have landed
        __syncthreads();
        if (s + 1 < n_steps) dma((s + 1) * kPK, lds_w1, lds_x1);
        compute(lds_w0, lds_x0);
        if (s + 1 < n_steps) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (s + 2 < n_steps) dma((s + 2) * kPK, lds_w0, lds_x0);
            compute(lds_w1, lds_x1);
        }
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
