// plx_backward.hip -- Parallax attention causal-prefill backward on gfx950
// (bf16 storage, fp32 accumulation).
//
// The forward is o_i = o^SA_i - Sigma^(i)_KV rho_i (the gist.science summary
// of Parallax, "Method: Parallax / core mechanism"; no boundary term, "key
// design choices").  Written as o_i = sum_j w_ij v_j with
// w_ij = p_ij (1 - r_ij + rbar_i), r_ij = rho_i . k_j, rbar_i = sum_j p_ij r_ij,
// its gradients for an upstream dO are
//
//   g_ij  = dO_i . v_j        G_i = dO_i . o^SA_i        D_i = dO_i . o_i + rbar_i G_i
//   dS_ij = p_ij (g_ij (1 - r_ij + rbar_i) + G_i r_ij - D_i)     (w.r.t. s = scale q.k)
//   dR_ij = p_ij (G_i - g_ij)                                    (w.r.t. r = rho.k)
//   dq_i = scale sum_j dS_ij k_j     drho_i = sum_j dR_ij k_j
//   dk_j = scale sum_i dS_ij q_i + sum_i dR_ij rho_i             dv_j = sum_i w_ij dO_i
//
// (derived: dL/dw_ij = g_ij; w depends on p, r and rbar; then the softmax).
// The pages train with this layer but print no backward pass.  With a zero
// probe these are FlashAttention's gradients (r = rbar = 0, G = D).
//
// Two kernels, FlashAttention-2 style, recomputing p from the forward's
// per-row log2-sum-exp instead of storing it:
//   bwd_dq_kernel       a workgroup of 8 wavefronts owns 128 query rows (as
//                       the forward) and streams K/V tiles; dq and drho come
//                       out of one transposed read of the K tile.  It also
//                       forms each row's (lse, 1 + rbar, G, -D) and keeps them in
//                       the workspace for the next kernel.
//   bwd_dkdv_kernel     a workgroup of 8 wavefronts owns 128 keys (16 per
//                       wavefront, held in registers) and streams 64-row
//                       tiles of q, rho and dO over the G query heads of the
//                       KV head, so dk and dv sum over the group in-kernel
//                       with no atomics.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16; lane l, col = l % 16, grp = l / 16):
// A row col holds contraction slots 8grp..8grp+7, B column col the same
// slots, C rows 4grp..4grp+3 of column col.  Slots are a free permutation as
// long as A and B agree: wherever a GEMM contracts over keys (dq) or query
// rows (dk, dv), slot e of lane group grp is element 4grp + (e & 3) +
// 16 (e >> 2) of the 32-slice, which is both how two 16-row C blocks land in
// a lane and what ds_read_b64_tr_b16 returns (see plx_prefill.hip).
#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

constexpr int kBwdWaves = 8;
constexpr int kBwdKT = 64;   // dq kernel: keys per LDS tile
constexpr int kBwdQR = 64;   // dk/dv kernel: query rows per LDS step
constexpr int kRowPad = 16;  // LDS row padding in elements (32 bytes; see the forward)
constexpr int kXcds = 8;     // MI355X: 8 accelerator complex dies, one L2 each

// Workgroup id -> (unit = (b, kv head), block index), blocks of a unit in
// ascending order.  Workgroup ids are dealt to the XCDs round-robin; when the
// units divide by 8, XCD x runs units x, x + 8, ... one after another, so the
// workgroups sharing a unit's streamed tensors sit behind the same L2.
__device__ __forceinline__ void block_order(int id, int n_units, int n_blk, int *unit, int *blk) {
    if (n_units % kXcds == 0) {
        const int xcd = id % kXcds, slot = id / kXcds;
        *blk = slot % n_blk;
        *unit = xcd + kXcds * (slot / n_blk);
    } else {
        *blk = id / n_units;
        *unit = id % n_units;
    }
}

// Runs item(id, odd) for this workgroup's items; odd marks the odd rounds
// of a persistent grid.  A grid smaller than the item
// count (a multiple of the 8 XCDs then, one workgroup per CU) is persistent:
// workgroup (xcd, c), c < ncu, takes in round r the slot r*ncu + c (r even)
// or r*ncu + ncu-1-c (r odd) of its XCD's slot list, so the long and short
// blocks of a unit pair up, and every slot is taken once.  Its output stores
// then drain while its next item starts, instead of holding the CU until they
// are acknowledged.  Items end with a bare barrier (the next item's first
// loads overwrite LDS the last step read; those reads have completed, their
// data fed the last products): a __syncthreads() would also wait for the
// stores.  A grid of one workgroup per item takes item blockIdx.x.
template <class F>
__device__ __forceinline__ void persistent_items(int n_items, F &&item) {
    const bool persist = static_cast<int>(gridDim.x) < n_items;
    const int xcd = blockIdx.x % kXcds, c = blockIdx.x / kXcds, ncu = gridDim.x / kXcds;
    for (int r = 0;; ++r) {
        const int id = persist ? xcd + kXcds * (r * ncu + ((r & 1) ? ncu - 1 - c : c))
                               : (r == 0 ? static_cast<int>(blockIdx.x) : n_items);
        if (id >= n_items) break;  // later rounds only hold larger slots
        item(id, persist && (r & 1));
        asm volatile("" ::: "memory");  // no memory access moves across the barrier
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

// ---------------------------------------------------------------------------
// dq, drho: per workgroup 8 wavefronts x 16 query rows, K/V tiles of 64 keys.
// ---------------------------------------------------------------------------
template <int D, int G, bool HAS_RHO>
__global__ __launch_bounds__(kBwdWaves *kWave, 2) void bwd_dq_kernel(BackwardParams p) {
    using S = uint16_t;
    constexpr int KT = kBwdKT;
    constexpr int PW = 16 / G;            // positions per wavefront
    constexpr int BQ = PW * kBwdWaves;    // positions per workgroup
    constexpr int KS = D / 32;
    constexpr int NKB = KT / 16;
    constexpr int NU = KT / 32;
    constexpr int DT = D / 16;
    constexpr int RS = D + kRowPad;       // LDS row stride of K and V tiles
    constexpr int NTHR = kBwdWaves * kWave;
    constexpr int KCH = KT * D / 8;       // 8-element chunks per tile
    constexpr int NKC = (KCH + NTHR - 1) / NTHR;
    constexpr bool FULL = KCH % NTHR == 0;
    static_assert(16 % G == 0, "group size must divide the wavefront's 16 rows");

    // TPB tiles per barrier, 2 TPB buffers: a barrier opens tiles j .. j + TPB - 1,
    // and tiles j + TPB .. j + 2 TPB - 1 are stored meanwhile into the buffers
    // of tiles j - TPB .. j - 1, whose readers all finished before that
    // barrier (as in the forward kernel).
    constexpr int TPB = 2;  // measured ~2% faster for this kernel than one tile per barrier
    constexpr int NBUF = 2 * TPB;
    __shared__ __attribute__((aligned(16))) S lds_k[NBUF][KT * RS];
    __shared__ __attribute__((aligned(16))) S lds_v[NBUF][KT * RS];

    // One work item (a workgroup's share of one launch in the
    // one-item-per-workgroup order), from its first loads to its stores.  In
    // the persistent loop below nothing derived from the lane index is
    // hoisted out of the item loop (it would stay live across the tile loop).
    auto run_item = [&](int id, bool /*odd round*/) __attribute__((always_inline)) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & (kWave - 1);
        const int wave = tid / kWave;
        const int col = lane & 15;
        const int grp = lane >> 4;

        int qb, unit;
        block_order(id, p.B * p.Hkv, p.n_qblk, &unit, &qb);
        qb = p.n_qblk - 1 - qb;  // longest first
        const int b = unit / p.Hkv;
        const int g = unit % p.Hkv;
        const int T_len = p.T;
        const int pos0 = qb * BQ;
        const int wpos0 = pos0 + wave * PW;
        const int wpos_last = wpos0 + PW - 1;
        const int key_end = min(pos0 + BQ, T_len);
        const int n_tiles = (key_end + KT - 1) / KT;

        const int64_t kv_base = (static_cast<int64_t>(b) * p.Hkv + g) * T_len * static_cast<int64_t>(D);
        const S *kg = static_cast<const S *>(p.k) + kv_base;
        const S *vg = static_cast<const S *>(p.v) + kv_base;

        // This lane's row: position wpos0 + col / G of query head g*G + col % G.
        const int pos = wpos0 + col / G;
        const int head = g * G + col % G;
        const int64_t row = (static_cast<int64_t>(b) * p.Hq + head) * T_len + min(pos, T_len - 1);
        const int64_t roff = row * D;
        Op8<BF16> qop[KS], dop[KS], rop[HAS_RHO ? KS : 1];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[s] = op8_load(static_cast<const S *>(p.q) + roff + 32 * s + 8 * grp);
            dop[s] = op8_load(static_cast<const S *>(p.dout) + roff + 32 * s + 8 * grp);
            if constexpr (HAS_RHO) rop[s] = op8_load(static_cast<const S *>(p.rho) + roff + 32 * s + 8 * grp);
        }
        // The row's statistics are formed here and kept for the dk/dv kernel:
        // lse and rbar from the training forward, G = dO . o^SA and
        // D = dO . o + rbar G.  Each lane holds 32 of the row's head dims (its
        // four lane groups together hold all of them); two exchanges across the
        // groups finish the dot products.
        float dot_o = 0.f, dot_sa = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const Op8<BF16> ov = op8_load(static_cast<const S *>(p.out) + roff + 32 * s + 8 * grp);
            Op8<BF16> sv;
            if constexpr (HAS_RHO) sv = op8_load(static_cast<const S *>(p.out_sa) + roff + 32 * s + 8 * grp);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t dw = dop[s].w[h], owd = ov.w[h];
                dot_o = fmaf(bf16_to_f32(dw & 0xffffu), bf16_to_f32(owd & 0xffffu), dot_o);
                dot_o = fmaf(bf16_to_f32(dw >> 16), bf16_to_f32(owd >> 16), dot_o);
                if constexpr (HAS_RHO) {
                    const uint32_t sw = sv.w[h];
                    dot_sa = fmaf(bf16_to_f32(dw & 0xffffu), bf16_to_f32(sw & 0xffffu), dot_sa);
                    dot_sa = fmaf(bf16_to_f32(dw >> 16), bf16_to_f32(sw >> 16), dot_sa);
                }
            }
        }
        dot_o += __shfl_xor(dot_o, 16);
        dot_o += __shfl_xor(dot_o, 32);
        if constexpr (HAS_RHO) {
            dot_sa += __shfl_xor(dot_sa, 16);
            dot_sa += __shfl_xor(dot_sa, 32);
        }
        const float lse = p.lse[row];
        const float rbar = HAS_RHO ? p.rbar[row] : 0.f;
        const float Gi = HAS_RHO ? dot_sa : dot_o;
        const float Di = HAS_RHO ? dot_o + rbar * Gi : dot_o;
        const float one_rbar = 1.f + rbar, neg_D = -Di;
        // Kept as (lse, 1 + rbar, G, -D): the forms the elementwise terms use.
        if (grp == 0 && pos < T_len) p.rowst[row] = make_float4(lse, 1.f + rbar, Gi, -Di);

        int g_off[NKC], l_off[NKC];
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = min(tid + n * NTHR, KCH - 1);
            g_off[n] = (c / (D / 8)) * D + (c % (D / 8)) * 8;
            l_off[n] = (c / (D / 8)) * RS + (c % (D / 8)) * 8;
        }
        Op8<BF16> kreg[NKC], vreg[NKC];
        auto load_tile = [&](int j) {
            const int key0 = j * KT;
#pragma unroll
            for (int n = 0; n < NKC; ++n) {
                const int c = tid + n * NTHR;
                if (FULL || c < KCH) {
                    if (key0 + KT <= T_len) {
                        kreg[n] = op8_load(kg + static_cast<int64_t>(key0) * D + g_off[n]);
                        vreg[n] = op8_load(vg + static_cast<int64_t>(key0) * D + g_off[n]);
                    } else {
                        const int kk = min(key0 + c / (D / 8), T_len - 1);
                        const int off = (c % (D / 8)) * 8;
                        kreg[n] = op8_load(kg + static_cast<int64_t>(kk) * D + off);
                        vreg[n] = op8_load(vg + static_cast<int64_t>(kk) * D + off);
                    }
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int n = 0; n < NKC; ++n)
                if (FULL || tid + n * NTHR < KCH) {
                    store_op8(&lds_k[buf][l_off[n]], kreg[n]);
                    store_op8(&lds_v[buf][l_off[n]], vreg[n]);
                }
        };

        f32x4 dqacc[DT], dracc[HAS_RHO ? DT : 1];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            dqacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (HAS_RHO) dracc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        load_tile(0);
        store_tile(0);
        if (TPB > 1 && n_tiles > 1) {
            load_tile(1);
            store_tile(1);
        }
        for (int j = 0; j < n_tiles; ++j) {
            const int buf = j & (NBUF - 1);
            if (j % TPB == 0) __syncthreads();
            const bool more = j + TPB < n_tiles;
            if (more) load_tile(j + TPB);
            const int key0 = j * KT;
            if (key0 <= wpos_last) {
                const S *kt = lds_k[buf];
                const S *vt = lds_v[buf];
                // S^T = K q^T, R^T = K rho^T, g^T = V dO^T: rows are keys, the
                // lane's column is its query row.
                f32x4 sacc[NKB], racc[HAS_RHO ? NKB : 1], gacc[NKB];
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, r = a, gg = a;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const Op8<BF16> kop = op8_load(kt + (16 * kb + col) * RS + 32 * s + 8 * grp);
                        const Op8<BF16> vop = op8_load(vt + (16 * kb + col) * RS + 32 * s + 8 * grp);
                        a = mma32(kop, qop[s], a);
                        if constexpr (HAS_RHO) r = mma32(kop, rop[s], r);
                        gg = mma32(vop, dop[s], gg);
                    }
                    sacc[kb] = a;
                    if constexpr (HAS_RHO) racc[kb] = r;
                    gacc[kb] = gg;
                }
                __builtin_amdgcn_s_setprio(0);

                const bool diag = key0 + KT - 1 > wpos0;
                const int rel = pos - key0 - 4 * grp;  // key > pos <=> offset > rel
                // dS / scale (the scale multiplies dq once, in the epilogue) and dR.
                float ds[NKB * 4], dr[HAS_RHO ? NKB * 4 : 1];
                // Causal mask, on the tiles that cross the diagonal only (wave-uniform):
                // a masked score becomes -inf, so its p is 0 (the scale is positive).
                if (diag) {
#pragma unroll
                    for (int e = 0; e < NKB * 4; ++e)
                        if (16 * (e >> 2) + (e & 3) > rel) sacc[e >> 2][e & 3] = -INFINITY;
                }
#pragma unroll
                for (int e = 0; e < NKB * 4; ++e) {
                    const int kb = e >> 2, i = e & 3;
                    const float pr = fast_exp2(fmaf(sacc[kb][i], p.scale_log2, -lse));
                    const float gv = gacc[kb][i];
                    if constexpr (HAS_RHO) {
                        const float rv = racc[kb][i];
                        ds[e] = pr * fmaf(gv, one_rbar - rv, fmaf(Gi, rv, neg_D));
                        dr[e] = pr * (Gi - gv);
                    } else {
                        ds[e] = pr * (gv + neg_D);
                    }
                }
                Op8<BF16> dsop[NU], drop[HAS_RHO ? NU : 1];
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    float w[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = ds[8 * u + e];
                    dsop[u] = op8_pack(w, BF16{});
                    if constexpr (HAS_RHO) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = dr[8 * u + e];
                        drop[u] = op8_pack(w, BF16{});
                    }
                }
                // dq^T += K^T dS^T and drho^T += K^T dR^T: the K tile read
                // transposed gives, to lane col, dim 16t + col of the keys in the
                // slot order of dsop.
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int u = 0; u < NU; ++u) {
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        const S *a = kt + (32 * u + 4 * grp + (col >> 2)) * RS + 16 * t + 4 * (col & 3);
                        const Op8<BF16> ktr = op8_load_tr(a, a + 16 * RS);
                        dqacc[t] = mma32(ktr, dsop[u], dqacc[t]);
                        if constexpr (HAS_RHO) dracc[t] = mma32(ktr, drop[u], dracc[t]);
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
            if (more) store_tile((j + TPB) & (NBUF - 1));
        }

        if (pos < T_len) {
            S *dq = static_cast<S *>(p.dq) + roff;
            S *drho = HAS_RHO ? static_cast<S *>(p.drho) + roff : nullptr;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = p.scale * dqacc[t][i];
                store4(dq + 16 * t + 4 * grp, y);
                if constexpr (HAS_RHO) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = dracc[t][i];
                    store4(drho + 16 * t + 4 * grp, y);
                }
            }
        }
    };  // run_item
    const int n_items = p.B * p.Hkv * p.n_qblk;
    persistent_items(n_items, run_item);
}

// ---------------------------------------------------------------------------
// dk, dv: per workgroup 8 wavefronts x 16 keys; steps of 64 query rows of the
// G heads (row r of KV head g is position r / G of query head g*G + r % G).
// ---------------------------------------------------------------------------
template <int D, int G, bool HAS_RHO>
__global__ __launch_bounds__(kBwdWaves *kWave, 2) void bwd_dkdv_kernel(BackwardParams p) {
    using S = uint16_t;
    constexpr int QR = kBwdQR;
    constexpr int KB = 16 * kBwdWaves;    // keys per workgroup
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int RS = D + kRowPad;
    constexpr int NTHR = kBwdWaves * kWave;
    constexpr int QCH = QR * D / 8;       // 8-element chunks per row tile
    constexpr int NQC = (QCH + NTHR - 1) / NTHR;
    constexpr bool QFULL = QCH % NTHR == 0;
    constexpr int NTEN = HAS_RHO ? 3 : 2; // q, dO (, rho)
    constexpr int NQB = QR / 16;          // 16-row blocks per step
    constexpr int NUQ = QR / 32;          // 32-row slices per step

    __shared__ __attribute__((aligned(16))) S lds_q[2][QR * RS];
    __shared__ __attribute__((aligned(16))) S lds_d[2][QR * RS];
    __shared__ __attribute__((aligned(16))) S lds_r[HAS_RHO ? 2 : 1][HAS_RHO ? QR * RS : 8];
    __shared__ float4 lds_st[2][QR];

    // One work item (a workgroup's share of one launch in the
    // one-item-per-workgroup order), from its first loads to its stores.  In
    // the persistent loop below nothing derived from the lane index is
    // hoisted out of the item loop (it would stay live across the tile loop).
    auto run_item = [&](int id, bool fwd) __attribute__((always_inline)) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & (kWave - 1);
        const int wave = tid / kWave;
        const int col = lane & 15;
        const int grp = lane >> 4;

        int kblk, unit;  // key block 0 sees every query row: it goes first
        block_order(id, p.B * p.Hkv, p.n_kblk, &unit, &kblk);
        const int b = unit / p.Hkv;
        const int g = unit % p.Hkv;
        const int T_len = p.T;
        const int k0 = kblk * KB;
        const int kw0 = k0 + 16 * wave;         // this wavefront's first key
        const int key = kw0 + col;              // this lane's key
        // Row indices of the KV group are 32-bit: the entry point rejects T G >= 2^31.
        const int rows_total = T_len * G;
        const int r0 = k0 * G;  // first row that can see key k0
        const int n_steps = (rows_total - r0 + QR - 1) / QR;
        // The concurrently running key blocks of one KV head should read the
        // same row tile at about the same time, so that it is fetched into L2
        // once.  Blocks that start together (the one-item grid, and the even
        // rounds of the persistent grid) walk the rows from the last one
        // backwards on a grid common to all key blocks (step s covers rows
        // rows_total - (s+1) QR .. rows_total - s QR - 1; rows before r0 in the
        // last step, negative ones included, are masked).  In the odd rounds of
        // the persistent grid, key block k starts when the block before it on
        // its CU, the mirror block 31 - k of the even round's order, ends: the
        // later k, the later the start, by about the QR G-row steps that
        // separate the blocks' first rows.  Those blocks walk forwards from
        // their first row r0 (step s covers rows r0 + s QR ..; rows from
        // rows_total on, in the last step, are masked), which lines them up
        // on the same rows at the same time.  Measured fetch for B=8, T=4096:
        // 0.55 GB, against 2.05 GB with backward walks in every round.
        auto step_row0 = [&](int step) { return fwd ? r0 + step * QR : rows_total - (step + 1) * QR; };

        const int64_t kv_base = (static_cast<int64_t>(b) * p.Hkv + g) * T_len * static_cast<int64_t>(D);
        // The wavefront's keys as the B operand (column = key): K[key][dims].
        Op8<BF16> kop[KS], vop[KS];
        {
            const int kk = min(key, T_len - 1);
            const S *kr = static_cast<const S *>(p.k) + kv_base + static_cast<int64_t>(kk) * D;
            const S *vr = static_cast<const S *>(p.v) + kv_base + static_cast<int64_t>(kk) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                kop[s] = op8_load(kr + 32 * s + 8 * grp);
                vop[s] = op8_load(vr + 32 * s + 8 * grp);
            }
        }

        // Row tile loader: thread tid moves chunks tid, tid + NTHR, ... of each tensor.
        Op8<BF16> stg[NQC][NTEN];
        float4 stst = make_float4(0.f, 0.f, 0.f, 0.f);
        // Loader rows: chunk n of this thread is row lrow of the step, 8-element
        // column chunk cc.  A step's first row rs0 is a multiple of G (rows_total
        // = T G and QR are), so row rs0 + lrow is position rs0 / G + lrow / G of
        // query head g G + lrow % G: the head is fixed, and only the position
        // moves, by QR / G per step.  Only the last step reaches below position 0
        // or past the sequence (rows that are masked); their loads are clamped
        // into it.
        static_assert(QR % 8 == 0 && QFULL, "loader rows");
        int64_t lbase[NQC];  // element offset of (head, position 0, column chunk)
        int lpos[NQC];       // lrow / G
#pragma unroll
        for (int n = 0; n < NQC; ++n) {
            const int c = tid + n * NTHR, lrow = c / (D / 8), cc = c % (D / 8);
            lbase[n] = (static_cast<int64_t>(b) * p.Hq + g * G + lrow % G) * T_len * static_cast<int64_t>(D) + cc * 8;
            lpos[n] = lrow / G;
        }
        const int64_t sbase = (static_cast<int64_t>(b) * p.Hq + g * G + tid % G) * T_len;  // row statistics, tid < QR
        const int spos = tid / G;
        auto load_step = [&](int step) {
            const int pos0 = step_row0(step) / G;  // exact: step_row0 is a multiple of G
#pragma unroll
            for (int n = 0; n < NQC; ++n) {
                const int64_t off = lbase[n] + static_cast<int64_t>(min(max(pos0 + lpos[n], 0), T_len - 1)) * D;
                stg[n][0] = op8_load(static_cast<const S *>(p.q) + off);
                stg[n][1] = op8_load(static_cast<const S *>(p.dout) + off);
                if constexpr (HAS_RHO) stg[n][2] = op8_load(static_cast<const S *>(p.rho) + off);
            }
            if (tid < QR) stst = p.rowst[sbase + min(max(pos0 + spos, 0), T_len - 1)];
        };
        auto store_step = [&](int buf) {
#pragma unroll
            for (int n = 0; n < NQC; ++n) {
                const int c = tid + n * NTHR;
                if (QFULL || c < QCH) {
                    const int lo = (c / (D / 8)) * RS + (c % (D / 8)) * 8;
                    store_op8(&lds_q[buf][lo], stg[n][0]);
                    store_op8(&lds_d[buf][lo], stg[n][1]);
                    if constexpr (HAS_RHO) store_op8(&lds_r[buf][lo], stg[n][2]);
                }
            }
            if (tid < QR) lds_st[buf][tid] = stst;
        };

        f32x4 dkacc[DT], dvacc[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            dkacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            dvacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        if (n_steps > 0) {
            load_step(0);
            store_step(0);
        }
        for (int step = 0; step < n_steps; ++step) {
            const int buf = step & 1;
            __syncthreads();
            const bool more = step + 1 < n_steps;
            if (more) load_step(step + 1);
            const int rs0 = step_row0(step);
            // Rows of this step reach position (rs0 + QR - 1) / G; the wavefront's
            // keys start at kw0.  Skip (wavefront-uniformly) when no row can see them.
            if ((rs0 + QR - 1) / G >= kw0 && kw0 < T_len) {
                const S *qt = lds_q[buf];
                const S *dt = lds_d[buf];
                const S *rt = HAS_RHO ? lds_r[buf] : nullptr;
                // S = q K^T, R = rho K^T, g = dO V^T: rows are query rows (NQB
                // 16-row blocks), the lane's column is its key.
                f32x4 sacc[NQB], racc[HAS_RHO ? NQB : 1], gacc[NQB];
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, r = a, gg = a;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const int off = (16 * qb + col) * RS + 32 * s + 8 * grp;
                        a = mma32(op8_load(qt + off), kop[s], a);
                        if constexpr (HAS_RHO) r = mma32(op8_load(rt + off), kop[s], r);
                        gg = mma32(op8_load(dt + off), vop[s], gg);
                    }
                    sacc[qb] = a;
                    if constexpr (HAS_RHO) racc[qb] = r;
                    gacc[qb] = gg;
                }
                __builtin_amdgcn_s_setprio(0);

                float w[4 * NQB], ds[4 * NQB], dr[HAS_RHO ? 4 * NQB : 1];
                // Causal mask, only on steps whose first row comes before the
                // wavefront's last key or before r0, or whose rows run past the
                // sequence (wavefront-uniform): a masked score becomes -inf, so its
                // p is 0 (the scale is positive).  Valid rows reach position T - 1
                // at most, so keys past the sequence fail the causal test too.
                if (rs0 < r0 || rs0 / G < kw0 + 15 || rs0 + QR > rows_total) {
#pragma unroll
                    for (int e = 0; e < 4 * NQB; ++e) {
                        const int r = rs0 + 16 * (e >> 2) + 4 * grp + (e & 3);
                        if (!(r >= r0 && r < rows_total && key <= static_cast<int>(static_cast<unsigned>(r) / G)))
                            sacc[e >> 2][e & 3] = -INFINITY;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4 * NQB; ++e) {
                    const int qb = e >> 2, i = e & 3;
                    const int lr = 16 * qb + 4 * grp + i;  // row within the step
                    const float4 st = lds_st[buf][lr];     // (lse, 1 + rbar, G, -D)
                    const float pr = fast_exp2(fmaf(sacc[qb][i], p.scale_log2, -st.x));
                    const float gv = gacc[qb][i];
                    if constexpr (HAS_RHO) {
                        const float rv = racc[qb][i];
                        const float f = st.y - rv;
                        w[e] = pr * f;
                        ds[e] = (p.scale * pr) * fmaf(gv, f, fmaf(st.z, rv, st.w));
                        dr[e] = pr * (st.z - gv);
                    } else {
                        w[e] = pr;
                        ds[e] = (p.scale * pr) * (gv + st.w);
                    }
                }
                Op8<BF16> wop[NUQ], dsop[NUQ], drop[HAS_RHO ? NUQ : 1];
#pragma unroll
                for (int u = 0; u < NUQ; ++u) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = w[8 * u + e];
                    wop[u] = op8_pack(x, BF16{});
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = ds[8 * u + e];
                    dsop[u] = op8_pack(x, BF16{});
                    if constexpr (HAS_RHO) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = dr[8 * u + e];
                        drop[u] = op8_pack(x, BF16{});
                    }
                }
                // dv^T += dO^T W, dk^T += q^T dS + rho^T dR: the row tiles read
                // transposed give, to lane col, dim 16t + col of the rows in the
                // slot order of wop/dsop/drop (slice u: rows 32u + 4grp + 0..3
                // and the same + 16).
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int u = 0; u < NUQ; ++u) {
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        const int off = (32 * u + 4 * grp + (col >> 2)) * RS + 16 * t + 4 * (col & 3);
                        dvacc[t] = mma32(op8_load_tr(dt + off, dt + off + 16 * RS), wop[u], dvacc[t]);
                        dkacc[t] = mma32(op8_load_tr(qt + off, qt + off + 16 * RS), dsop[u], dkacc[t]);
                        if constexpr (HAS_RHO)
                            dkacc[t] = mma32(op8_load_tr(rt + off, rt + off + 16 * RS), drop[u], dkacc[t]);
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
            if (more) store_step(buf ^ 1);
        }

        if (key < T_len) {
            const int64_t off = kv_base + static_cast<int64_t>(key) * D;
            S *dk = static_cast<S *>(p.dk) + off;
            S *dv = static_cast<S *>(p.dv) + off;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = dkacc[t][i];
                store4(dk + 16 * t + 4 * grp, y);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = dvacc[t][i];
                store4(dv + 16 * t + 4 * grp, y);
            }
        }
    };  // run_item
    const int n_items = p.B * p.Hkv * p.n_kblk;
    persistent_items(n_items, run_item);
}

template <int D, int G, bool R>
hipError_t launch_bwd_r(const BackwardParams &p, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(p.B) * p.Hkv;
    // Persistent grids: one workgroup per CU, a multiple of the 8 XCDs.
    const int64_t grid = device_cus() / kXcds * kXcds;
    int64_t dq_blocks = units * p.n_qblk;
    if (grid > 0 && dq_blocks > grid) dq_blocks = grid;
    hipLaunchKernelGGL((bwd_dq_kernel<D, G, R>), dim3(static_cast<uint32_t>(dq_blocks)),
                       dim3(kBwdWaves * kWave), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t kv_blocks = units * p.n_kblk;
    if (grid > 0 && kv_blocks > grid) kv_blocks = grid;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, G, R>), dim3(static_cast<uint32_t>(kv_blocks)),
                       dim3(kBwdWaves * kWave), 0, stream, p);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_bwd_g(const BackwardParams &p, hipStream_t stream) {
    return p.rho ? launch_bwd_r<D, G, true>(p, stream) : launch_bwd_r<D, G, false>(p, stream);
}

template <int D>
hipError_t launch_bwd_d(const BackwardParams &p, int G, hipStream_t stream) {
    switch (G) {
    case 1: return launch_bwd_g<D, 1>(p, stream);
    case 2: return launch_bwd_g<D, 2>(p, stream);
    case 4: return launch_bwd_g<D, 4>(p, stream);
    case 8: return launch_bwd_g<D, 8>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int backward_q_block_positions(int G) { return 16 / G * kBwdWaves; }
int backward_k_block_keys() { return 16 * kBwdWaves; }

hipError_t launch_backward(const BackwardParams &p, int D, int G, hipStream_t stream) {
    switch (D) {
    case 64: return launch_bwd_d<64>(p, G, stream);
    case 128: return launch_bwd_d<128>(p, G, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace plx
