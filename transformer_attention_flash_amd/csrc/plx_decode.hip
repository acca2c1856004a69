// plx_decode.hip -- Parallax attention decode on gfx950: split-KV kernel and
// the kernel that merges the splits.
//
// One workgroup of 1, 2 or 4 wavefronts owns one (sequence b, KV head g,
// key chunk) work item; its wavefronts take interleaved 32-key tiles of the
// chunk and merge their states in LDS at the end.  The G query heads that
// share KV head g and their G probes form the 2G columns of a 16-column MFMA
// tile: columns 0..G-1 are the query rows, columns G..2G-1
// the probe rows, the rest are zero.  One MFMA over a 16-key block of K
// therefore gives the softmax scores S = tau q.k and the probe scores
// R = rho.k together, and one MFMA over 32 keys of V gives the softmax
// numerator A = sum P v and the probe-weighted numerator B = sum (P r) v in
// the same tile.  The probe rows fill MFMA columns that a query-only decode
// would leave empty, so the correction branch costs no extra matrix
// instructions and no extra K/V traffic (the news.chathome.org article on
// Parallax, "Hardware argument": both branches share the K/V tiles and the
// online max and scaling factors; the gist.science summary, "Hardware-aware
// algorithm": QK and RK products inside the same matrix instructions).
//
// Orientation: the kernel computes S^T = K [q; rho]^T (keys along M) and
// O^T = V^T [P; P*R]^T, so that each lane ends up owning one column (one
// query or probe row) and the softmax state of that row needs no transpose
// between the two MFMAs.  The value operand wants 8 keys of one head
// dimension per lane; each lane loads 8 key rows (contiguous across the
// wavefront) and transposes its 8 x (d/16) block in registers.
//
// Per-row state (m, l, c, A, B): m is the running max of the scaled scores in
// log2 units, l = sum P, c = sum P r, A = sum P v, B = sum P r v with
// P = 2^(s*log2e - m).  The epilogue forms o = A/l - (B/l - (c/l) A/l).
#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

constexpr float kRescaleSlack = 8.f;
constexpr int kCombineWaves = 4;  // wavefronts merging one (sequence, query head) row

// The d/16 head-dimension elements a lane reads from one value row.
template <class T, int CH> struct VChunk;
template <int CH> struct VChunk<BF16, CH> {
    uint32_t w[CH / 2];
};
template <int CH> struct VChunk<F32, CH> {
    float v[CH];
};

template <int CH>
__device__ __forceinline__ VChunk<BF16, CH> vchunk_load(const uint16_t *p) {
    VChunk<BF16, CH> c;
    if constexpr (CH == 8) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));  // streamed once
#pragma unroll
        for (int j = 0; j < 4; ++j) c.w[j] = x[j];
    } else {
        static_assert(CH == 4, "value chunk");
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        c.w[0] = x[0];
        c.w[1] = x[1];
    }
    return c;
}
template <int CH>
__device__ __forceinline__ VChunk<F32, CH> vchunk_load(const float *p) {
    VChunk<F32, CH> c;
#pragma unroll
    for (int j = 0; j < CH / 4; ++j) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) c.v[4 * j + e] = x[e];
    }
    return c;
}

// Value operand of MFMA t: element t of the 8 loaded key rows, in slot order.
template <int CH>
__device__ __forceinline__ Op8<BF16> value_op(const VChunk<BF16, CH> (&vr)[8], int t) {
    Op8<BF16> o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o.w[j] = half_lo(vr[2 * j].w[t >> 1], t) | half_hi(vr[2 * j + 1].w[t >> 1], t);
    return o;
}
template <int CH>
__device__ __forceinline__ Op8<F32> value_op(const VChunk<F32, CH> (&vr)[8], int t) {
    Op8<F32> o;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) o.v[kk] = vr[kk].v[t];
    return o;
}

__device__ __forceinline__ void store_chunk(uint16_t *dst, const float *x, int n) {
    // n is 4 or 8 contiguous outputs
    if (n == 8) {
        *reinterpret_cast<u32x4 *>(dst) =
            u32x4{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]),
                  pack2_bf16(x[6], x[7])};
    } else {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3])};
    }
}
__device__ __forceinline__ void store_chunk(float *dst, const float *x, int n) {
    for (int j = 0; j < n / 4; ++j)
        reinterpret_cast<f32x4 *>(dst)[j] = f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}

struct SeqView {
    int64_t start;  // token offset of the sequence in the cache
    int64_t len;    // number of cached keys
};

__device__ __forceinline__ SeqView seq_view(const DecodeParams &p, int b) {
    SeqView s;
    if (p.cu) {
        s.start = p.cu[b];
        s.len = p.cu[b + 1] - s.start;
    } else {
        s.start = static_cast<int64_t>(b) * p.max_ctx;
        s.len = p.max_ctx;
    }
    return s;
}

}  // namespace

template <class T, int D, int G, int NW>
__global__ __launch_bounds__(NW *kWave) void decode_split_kernel(DecodeParams p) {
    using S = typename T::storage;
    constexpr int KS = D / 32;  // 32-wide contraction slices over the head dim
    constexpr int CH = D / 16;  // head-dim elements per lane in the value operand
    static_assert(2 * G <= 16, "query + probe rows must fit 16 MFMA columns");

    // Wavefronts of the workgroup take interleaved 32-key tiles of the chunk
    // and merge their softmax states through LDS at the end.
    __shared__ float s_m[NW > 1 ? NW : 1][16];
    __shared__ float s_l[NW > 1 ? NW : 1][16];
    __shared__ __attribute__((aligned(16))) float s_acc[NW > 1 ? NW : 1][CH * 4][kWave];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int64_t item = blockIdx.x;
    const int split = static_cast<int>(item % p.n_split);
    const int64_t unit = item / p.n_split;
    const int b = static_cast<int>(unit / p.Hkv);
    const int g = static_cast<int>(unit % p.Hkv);

    const SeqView sv = seq_view(p, b);
    const int64_t k_begin = static_cast<int64_t>(split) * p.keys_per_split;
    if (k_begin >= sv.len) {
        // Nothing to read.  With a single split this kernel also owns the
        // output, and an empty sequence returns zeros.
        if (p.n_split == 1 && wave == 0) {
            S *o = static_cast<S *>(p.out) + (static_cast<int64_t>(b) * p.Hq + g * G) * D;
            for (int e = lane; e < G * D; e += kWave) o[e] = to_storage(0.f, T{});
        }
        return;
    }
    const int64_t k_end = min(k_begin + static_cast<int64_t>(p.keys_per_split), sv.len);
    const int64_t last = k_end - 1;

    const bool is_q = col < G;
    const bool is_r = !is_q && col < 2 * G;
    const int head = g * G + (is_q ? col : col - G);
    const int64_t row = static_cast<int64_t>(b) * p.Hq + head;

    // B operand: this lane's column of [q; rho], slices 32*s + 8*grp .. +7.
    const S *src = nullptr;
    if (is_q) src = static_cast<const S *>(p.q) + row * D;
    else if (is_r && p.rho) src = static_cast<const S *>(p.rho) + row * D;
    Op8<T> qop[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = src ? op8_load(src + 32 * s + 8 * grp) : op8_zero(T{});

    const int64_t kv0 = (sv.start * p.Hkv + static_cast<int64_t>(g) * sv.len) * D;
    const S *kbase = static_cast<const S *>(p.k) + kv0;
    const S *vbase = static_cast<const S *>(p.v) + kv0;
    const float sc = is_q ? p.scale_log2 : 1.f;

    float m_run = -INFINITY;
    float rsum = 0.f;  // l on query columns, c on probe columns (this lane's keys)
    f32x4 acc[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Each iteration covers SUB 32-key sub-tiles whose loads are all issued
    // before any is used, so a wavefront keeps 16 KB of K/V in flight at
    // either head dimension (d = 64 rows are half as long).
    constexpr int SUB = D == 64 ? 2 : 1;
    for (int64_t kt0 = k_begin + 32 * SUB * wave; kt0 < k_end; kt0 += 32 * SUB * NW) {
        // K: A operand rows are keys kt + 16*blk + col (clamped into the chunk;
        // clamped keys are masked below).
        Op8<T> kop[SUB][2][KS];
        // V: slot kk of this lane is key kt + 16*(kk/4) + 4*grp + kk%4, the
        // same key the score tile hands this lane in C position (kk/4, kk%4).
        VChunk<T, CH> vr[SUB][8];
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
            const int64_t kt = kt0 + 32 * sb;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int64_t key = min(kt + 16 * blk + col, last);
#pragma unroll
                for (int s = 0; s < KS; ++s) kop[sb][blk][s] = op8_load_stream(kbase + key * D + 32 * s + 8 * grp);
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int64_t key = min(kt + 16 * (kk >> 2) + 4 * grp + (kk & 3), last);
                vr[sb][kk] = vchunk_load<CH>(vbase + key * D + CH * col);
            }
        }

#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
            const int64_t kt = kt0 + 32 * sb;
            // [S; R]^T for 32 keys.
            f32x4 sr[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                sr[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) sr[blk] = mma32(kop[sb][blk][s], qop[s], sr[blk]);
            }

            float x[8];
            float mt = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t key = kt + 16 * (e >> 2) + 4 * grp + (e & 3);
                float v = sr[e >> 2][e & 3] * sc;
                if (is_q && key > last) v = -INFINITY;
                x[e] = v;
                mt = fmaxf(mt, v);
            }
            // The running max only moves when some query column's tile max
            // exceeds it by more than kRescaleSlack (log2 units): P stays below
            // 2^slack, and the rescale of l, c, A, B is rare.  The decision is
            // wave-uniform; the cross-lane row max is only formed when it fires.
            const bool grow = wave_any(is_q && mt > m_run + kRescaleSlack);
            float alpha_own = 1.f;
            if (grow) {
                mt = group_max(mt);
                const float m_new = fmaxf(m_run, mt);
                alpha_own = fast_exp2(m_run - m_new);
                m_run = m_new;
            }

            float pq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pq[e] = fast_exp2(x[e] - m_run);
            // Probe columns take the probabilities and the rescale factor of the
            // query column of the same head, G lanes to their left.
            const float alpha_q = row_shr<G>(alpha_own);
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pf = row_shr<G>(pq[e]);
                pv[e] = is_q ? pq[e] : (is_r ? pf * x[e] : 0.f);
            }
            const float alpha = is_q ? alpha_own : (is_r ? alpha_q : 1.f);
            const Op8<T> pop = op8_pack(pv, T{});
            if (grow) {
                rsum *= alpha;
#pragma unroll
                for (int t = 0; t < CH; ++t) acc[t] *= alpha;
            }
            rsum = op8_sum_acc(pop, rsum);

#pragma unroll
            for (int t = 0; t < CH; ++t) acc[t] = mma32(value_op<CH>(vr[sb], t), pop, acc[t]);
        }
    }

    rsum = group_sum(rsum);

    if constexpr (NW > 1) {
        // Probe columns are weighted by the max of their query column.  The
        // lane shift runs on every lane (its source lanes must be active).
        const float m_q = row_shr<G>(m_run);
        const float m_eff = is_r ? m_q : m_run;
        if (grp == 0) {
            s_m[wave][col] = m_eff;
            s_l[wave][col] = rsum;
        }
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc[wave][4 * t + i][lane] = acc[t][i];
        __syncthreads();
        if (wave != 0) return;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][col]);
        rsum = 0.f;
#pragma unroll
        for (int t = 0; t < CH; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            // A wavefront that saw no keys has m = -inf and weight 0.
            const float wt = fast_exp2(s_m[w][col] - M);
            rsum += wt * s_l[w][col];
#pragma unroll
            for (int t = 0; t < CH; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][i] += wt * s_acc[w][4 * t + i][lane];
        }
        // Only the query columns' m is read below (partials); probe columns
        // carry the query column's weights already.
        m_run = M;
    }

    // acc[t][i] of this lane is head-dim CH*(4*grp + i) + t of its column.
    if (p.n_split == 1) {
        const float l_q = row_shr<G>(rsum);
        float aq[CH][4];
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) aq[t][i] = row_shr<G>(acc[t][i]);
        if (is_r) {
            const float inv = 1.f / l_q;
            const float cbar = rsum * inv;
            S *o = static_cast<S *>(p.out) + row * D;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y[CH];
#pragma unroll
                for (int t = 0; t < CH; ++t) {
                    const float osa = aq[t][i] * inv;
                    const float corr = acc[t][i] * inv - cbar * osa;
                    y[t] = osa - corr;
                }
                store_chunk(o + CH * (4 * grp + i), y, CH);
            }
        }
    } else if (is_q || is_r) {
        const int64_t slot = row * p.n_split + split;
        if (grp == 0) {
            if (is_q) {
                p.ws_stats[slot * 3 + 0] = m_run;
                p.ws_stats[slot * 3 + 1] = rsum;
            } else {
                p.ws_stats[slot * 3 + 2] = rsum;
            }
        }
        float *dst = p.ws_vec + (slot * 2 + (is_q ? 0 : 1)) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float y[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) y[t] = acc[t][i];
            store_chunk(dst + CH * (4 * grp + i), y, CH);
        }
    }
}

// Merge the chunks of one (b, query head) row: M = max m_s, w_s = 2^(m_s - M),
// then (l, c, A, B) = sum_s w_s (l_s, c_s, A_s, B_s) in chunk order, and the
// same epilogue as the single-chunk path.
template <class T, int D>
__global__ __launch_bounds__(kCombineWaves *kWave) void decode_combine_kernel(DecodeParams p) {
    using S = typename T::storage;
    constexpr int PER = D / kWave;  // head-dim elements per lane
    constexpr int NW = kCombineWaves;
    __shared__ float s_red[NW][2 + 2 * D];  // per wavefront: l, c, A[D], B[D]
    __shared__ float s_max[NW];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int64_t row = blockIdx.x;
    const int b = static_cast<int>(row / p.Hq);
    S *o = static_cast<S *>(p.out) + row * D;

    const SeqView sv = seq_view(p, b);
    if (sv.len <= 0) {
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < PER; ++e) o[lane * PER + e] = to_storage(0.f, T{});
        }
        return;
    }
    const int64_t n64 = (sv.len + p.keys_per_split - 1) / p.keys_per_split;
    const int n = static_cast<int>(min(n64, static_cast<int64_t>(p.n_split)));
    const float *st = p.ws_stats + row * p.n_split * 3;

    // M = max over the splits' m: every thread takes a strided share, then
    // a wavefront and a workgroup reduction (max is exact in any order).
    float M = -INFINITY;
    for (int s = threadIdx.x; s < n; s += NW * kWave) M = fmaxf(M, st[3 * s]);
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
    if (lane == 0) s_max[wave] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_max[w]);

    // Wavefront w sums splits w, w + NW, ... in that order; its loop is
    // unrolled so that several splits' loads are in flight at once.
    float l = 0.f, c = 0.f, a[PER], bb[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = bb[e] = 0.f;
#pragma unroll 4
    for (int s = wave; s < n; s += NW) {
        const float w = fast_exp2(st[3 * s] - M);
        l += w * st[3 * s + 1];
        c += w * st[3 * s + 2];
        const float *va = p.ws_vec + ((row * p.n_split + s) * 2) * D + lane * PER;
        const float *vb = va + D;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            a[e] += w * va[e];
            bb[e] += w * vb[e];
        }
    }
    // The wavefronts' partial sums are added in wavefront order.
    if (lane == 0) {
        s_red[wave][0] = l;
        s_red[wave][1] = c;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        s_red[wave][2 + lane * PER + e] = a[e];
        s_red[wave][2 + D + lane * PER + e] = bb[e];
    }
    __syncthreads();
    if (wave != 0) return;
    l = 0.f;
    c = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = bb[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        l += s_red[w][0];
        c += s_red[w][1];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            a[e] += s_red[w][2 + lane * PER + e];
            bb[e] += s_red[w][2 + D + lane * PER + e];
        }
    }
    const float inv = 1.f / l;
    const float cbar = c * inv;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const float osa = a[e] * inv;
        const float corr = bb[e] * inv - cbar * osa;
        o[lane * PER + e] = to_storage(osa - corr, T{});
    }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

namespace {

// Wavefronts per workgroup: one per 128 keys of the chunk, at most 4.  A CU
// holds two such workgroups at d = 128 (180 VGPRs) and three at d = 64 (168),
// but only one of 8 wavefronts; 8-wavefront workgroups measured 0.5-5%
// slower on chunks of 1024 keys and more (5% at d = 64).
template <class T, int D, int G, int NW>
void launch_split(const DecodeParams &p, int64_t items, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, NW>), dim3(static_cast<uint32_t>(items)), dim3(NW * kWave), 0,
                       stream, p);
}

template <class T, int D, int G>
hipError_t launch_decode_g(const DecodeParams &p, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(p.B) * p.Hkv * p.n_split;
    if (p.keys_per_split >= 512) launch_split<T, D, G, 4>(p, items, stream);
    else if (p.keys_per_split >= 256) launch_split<T, D, G, 2>(p, items, stream);
    else launch_split<T, D, G, 1>(p, items, stream);
    if (p.n_split > 1) {
        const int64_t rows = static_cast<int64_t>(p.B) * p.Hq;
        hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(static_cast<uint32_t>(rows)),
                           dim3(kCombineWaves * kWave), 0, stream, p);
    }
    return hipGetLastError();
}

template <class T, int D>
hipError_t launch_decode_d(const DecodeParams &p, int G, hipStream_t stream) {
    switch (G) {
    case 1: return launch_decode_g<T, D, 1>(p, stream);
    case 2: return launch_decode_g<T, D, 2>(p, stream);
    case 4: return launch_decode_g<T, D, 4>(p, stream);
    case 8: return launch_decode_g<T, D, 8>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t launch_decode_t(const DecodeParams &p, int D, int G, hipStream_t stream) {
    switch (D) {
    case 64: return launch_decode_d<T, 64>(p, G, stream);
    case 128: return launch_decode_d<T, 128>(p, G, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, bool bf16, int D, int G, hipStream_t stream) {
    return bf16 ? launch_decode_t<BF16>(p, D, G, stream) : launch_decode_t<F32>(p, D, G, stream);
}

}  // namespace plx
