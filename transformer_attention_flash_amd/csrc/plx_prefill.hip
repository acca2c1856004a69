// plx_prefill.hip -- causal Parallax attention prefill on gfx950.
//
// A workgroup of 8 wavefronts owns one (sequence b, KV head g, query block)
// tile: 128 query rows = the G query heads that share KV head g at 128/G
// consecutive positions.  Each wavefront owns 16 of those rows as one
// 16-column MFMA tile.  K/V tiles of KT keys are staged once in LDS (two
// or, for bf16 with the probe, four buffers) and shared by every row of the
// workgroup and by both scoring branches (the news.chathome.org article on Parallax, "Hardware
// argument": the two branches share the online max, the scaling factors and
// the K and V tiles; the gist.science summary, "Hardware-aware algorithm").
//
// Per key tile and 16-row column tile a wavefront issues
//   S^T = K q^T and R^T = K rho^T       (the same K operand registers),
//   A^T += V^T P^T and B^T += V^T (P*R)^T (the same V operand registers),
// with P = 2^(s*log2e - m) from the running max m of the query row, shared
// by the probe branch, and the same rescale factor applied to A, B, l and c.
// The probe rows thus ride in the same MFMA stream as the query rows (the
// probe tile is the query tile's neighbour in the N dimension); the softmax
// state is computed once.  The epilogue forms o = A/l - (B/l - (c/l) A/l).
//
// LDS layouts:
//   K  [KT][D + 32 B] natural rows; a lane's A operand is 8 contiguous dims.
//   V (bf16) [KT][D + pad] natural rows, read with the gfx950 transposing LDS
//                     load ds_read_b64_tr_b16: two of them give a lane the 8
//                     keys of one head dimension that a value operand needs.
//   Vt (fp32) [D][KT + pad] transposed, with the keys of each 32-key slice
//                     permuted so that the 8 keys a lane needs for one value
//                     operand are contiguous: key 16*blk + 4*q + i (blk = 16-key
//                     block of the score tile, q = lane group, i = C-tile row)
//                     sits at position 32*(blk/2) + 8*q + 4*(blk%2) + i.  The
//                     loader transposes 4-key x 8-dim blocks in registers.
// The softmax-only kernel (no probe) is the same template with the probe
// branch compiled out; it runs the query-side arithmetic in the same order,
// so a zero probe reproduces its output bit for bit.
#include <atomic>
#include <type_traits>

#include "plx_device.h"
#include "plx_kernels.h"

namespace plx {

namespace {

template <class T> struct PrefillCfg;
template <> struct PrefillCfg<BF16> {
    static constexpr int KT = 64;  // keys per LDS tile
};
template <> struct PrefillCfg<F32> {
    static constexpr int KT = 32;
};

constexpr int kPrefillWaves = 8;
constexpr int kColTiles = 1;  // 16-row column tiles per wavefront
constexpr float kRescaleSlack = 8.f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// Reductions over the four lane groups (16-lane rows) that hold the same
// column, by the gfx950 row swaps: v_permlane16_swap with both operands x
// returns (x of row 2k, x of row 2k + 1) to both rows of each pair, and
// v_permlane32_swap (x of rows 0-1, x of rows 2-3) to both halves, so every
// lane combines the same two values in the same order, as the lane-shuffle
// forms do, without their LDS round trip.  Call them with every lane active.
// (The decode kernel keeps the shuffle forms: its short-context case measured
// 2% slower with these.)
__device__ __forceinline__ float row_group_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_group_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Four Op8 rows (keys 4r .. 4r+3 of one 8-dim chunk) -> element e of each, as
// the 4 contiguous LDS entries of transposed row e.
__device__ __forceinline__ void store_vt4(uint16_t *dst, const Op8<BF16> (&v)[4], int e) {
    const uint32_t w0 = half_lo(v[0].w[e >> 1], e) | half_hi(v[1].w[e >> 1], e);
    const uint32_t w1 = half_lo(v[2].w[e >> 1], e) | half_hi(v[3].w[e >> 1], e);
    *reinterpret_cast<u32x2 *>(dst) = u32x2{w0, w1};
}
__device__ __forceinline__ void store_vt4(float *dst, const Op8<F32> (&v)[4], int e) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0].v[e], v[1].v[e], v[2].v[e], v[3].v[e]};
}

}  // namespace

template <class T, int D, int G, bool HAS_RHO>
__global__ __launch_bounds__(kPrefillWaves *kWave, 2) void prefill_kernel(PrefillParams p) {
    using S = typename T::storage;
    constexpr int KT = PrefillCfg<T>::KT;
    constexpr int NB = kColTiles;
    constexpr int PW = 16 * NB / G;          // positions per wavefront
    constexpr int BQ = PW * kPrefillWaves;   // positions per workgroup
    constexpr int KS = D / 32;               // contraction slices over the head dim
    constexpr int NKB = KT / 16;             // 16-key blocks per tile
    constexpr int NU = KT / 32;              // 32-key slices for the value GEMMs
    constexpr int DT = D / 16;               // 16-dim output tiles
    constexpr int PAD = 16 / sizeof(S);      // one 16-byte bank group of padding
    // K rows carry 32 bytes of padding: with 16 the 16-byte operand reads of
    // consecutive key rows hit the same banks in pairs (measured); with 32
    // they are conflict-free and so are the tile stores.
    constexpr int KRS = D + 32 / sizeof(S);  // K row stride (elements)
    constexpr int VRS = KT + PAD;            // Vt row stride (elements), transposed layout
    // bf16 V stays in natural [key][dim] rows and is read transposed by
    // ds_read_b64_tr_b16; 16 extra elements per row put the 4 key rows one
    // transposed read touches in distinct banks.
    constexpr bool VNAT = std::is_same<T, BF16>::value;
    constexpr int VNRS = D + 16;             // V row stride (elements), natural layout
    constexpr int NTHR = kPrefillWaves * kWave;
    constexpr int KCH = KT * D / 8;          // 8-element K chunks per tile
    constexpr int NKC = (KCH + NTHR - 1) / NTHR;
    constexpr int VRUN = (KT / 4) * (D / 8); // 4-key x 8-dim V blocks per tile
    constexpr int NVR = (VRUN + NTHR - 1) / NTHR;
    static_assert(16 * NB % G == 0, "group size must divide the wave's rows");

    // TPB tiles per barrier, 2 * TPB tile buffers: a barrier opens tiles
    // j .. j + TPB - 1, and tiles j + TPB .. j + 2 TPB - 1 are stored meanwhile
    // into the buffers of tiles j - TPB .. j - 1, whose readers all finished
    // before that barrier.  bf16 with a probe: 2 (measured 3% faster); the
    // softmax-only kernel measured 12% slower that way and keeps 1.
    constexpr int TPB = (VNAT && HAS_RHO) ? 2 : 1;
    // bf16 with a probe runs a persistent grid (one workgroup per CU, which
    // is all the registers allow): a workgroup's output stores then drain
    // while its next item starts, instead of holding the CU until they are
    // acknowledged, and the next item's q / rho loads are issued during the
    // current item's last tile (measured 3-4% faster together).  The
    // softmax-only kernel fits two workgroups per CU, which hide each other's
    // ends, and keeps one item per workgroup.
    constexpr bool PERSIST = VNAT && HAS_RHO;
    constexpr int NBUF = 2 * TPB;
    __shared__ __attribute__((aligned(16))) S lds_k[NBUF][KT * KRS];
    __shared__ __attribute__((aligned(16))) S lds_v[NBUF][VNAT ? KT * VNRS : D * VRS];

    const int n_units = p.B * p.Hkv;

    // Item id -> (query block, unit).  Workgroups are dealt to the 8 XCDs
    // round-robin by id, and each XCD has its own 4 MB L2.  When the
    // (b, kv head) units divide evenly, XCD x runs units x, x + 8, ... one
    // after another, each with its query blocks longest first: the CUs of an
    // XCD then stream the same unit's K/V (2 MB at T = 4096, d = 128)
    // together, so it is fetched into L2 about once instead of once per
    // query block.
    auto item_of = [&](int id, int &qb, int &unit) __attribute__((always_inline)) {
        if (n_units % kXcds == 0) {
            const int xcd = id % kXcds, slot = id / kXcds;
            qb = p.n_qblk - 1 - slot % p.n_qblk;
            unit = xcd + kXcds * (slot / p.n_qblk);
        } else {  // longest query blocks first
            qb = p.n_qblk - 1 - id / n_units;
            unit = id % n_units;
        }
    };
    // The q and rho operands of this lane's rows in item id: column tile nb,
    // column col -> row r = 16*nb + col of the wavefront, position
    // wpos0 + r / G, query head g*G + r % G.
    auto load_rows = [&](int id, int wave, int col, int grp, Op8<T> (&q)[NB][KS],
                         Op8<T> (&rr)[NB][HAS_RHO ? KS : 1]) __attribute__((always_inline)) {
        int qb, unit;
        item_of(id, qb, unit);
        const int b = unit / p.Hkv, g = unit % p.Hkv;
        const int wpos0 = qb * BQ + wave * PW;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int r = 16 * nb + col;
            const int head = g * G + r % G;
            const int64_t off = ((static_cast<int64_t>(b) * p.Hq + head) * p.T + min(wpos0 + r / G, p.T - 1)) * D;
            const S *qrow = static_cast<const S *>(p.q) + off;
#pragma unroll
            for (int s = 0; s < KS; ++s) q[nb][s] = op8_load(qrow + 32 * s + 8 * grp);
            if constexpr (HAS_RHO) {
                const S *rrow = static_cast<const S *>(p.rho) + off;
#pragma unroll
                for (int s = 0; s < KS; ++s) rr[nb][s] = op8_load(rrow + 32 * s + 8 * grp);
            }
        }
    };
    // Persistent grid: the next item's q and rho operands, requested during
    // the current item's last tile (after its last score products, when the
    // current operands are dead), so that their memory latency runs under
    // that tile's softmax and value products and the epilogue.
    Op8<T> nq[NB][KS];
    Op8<T> nr[NB][HAS_RHO ? KS : 1];

    // One work item: item `id` of the grid order below, from its first K/V
    // tile to its output rows; `next` is the item to request operands for.
    auto run_item = [&](int id, int next) __attribute__((always_inline)) {
        int tid = threadIdx.x;
        // In the persistent loop nothing derived from the lane index is hoisted
        // out of the item loop (the hoisted values would stay live across the
        // tile loop and push it past the register budget).
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int lane = tid & (kWave - 1);
        const int wave = tid / kWave;
        const int col = lane & 15;
        const int grp = lane >> 4;

        int qb, unit;
        item_of(id, qb, unit);
        const int b = unit / p.Hkv;
        const int g = unit % p.Hkv;
        const int T_len = p.T;

        const int pos0 = qb * BQ;
        const int wpos0 = pos0 + wave * PW;
        const int wpos_last = wpos0 + PW - 1;
        const int key_end = min(pos0 + BQ, T_len);  // keys this workgroup ever needs
        const int n_tiles = (key_end + KT - 1) / KT;

        const int64_t kv_base = (static_cast<int64_t>(b) * p.Hkv + g) * T_len * static_cast<int64_t>(D);
        const S *kg = static_cast<const S *>(p.k) + kv_base;
        const S *vg = static_cast<const S *>(p.v) + kv_base;

        // This lane's rows: column tile nb, column col -> row r = 16*nb + col of
        // the wavefront, position wpos0 + r / G, query head g*G + r % G.
        int pos[NB];
        int64_t qoff[NB];
        Op8<T> qop[NB][KS];
        Op8<T> rop[NB][HAS_RHO ? KS : 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int r = 16 * nb + col;
            pos[nb] = wpos0 + r / G;
            const int head = g * G + r % G;
            qoff[nb] = ((static_cast<int64_t>(b) * p.Hq + head) * T_len + min(pos[nb], T_len - 1)) * D;
        }
        if constexpr (PERSIST) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    qop[nb][s] = nq[nb][s];
                    if constexpr (HAS_RHO) rop[nb][s] = nr[nb][s];
                }
        } else {
            load_rows(id, wave, col, grp, qop, rop);
        }

        // Loader registers for one tile.
        Op8<T> kreg[NKC];
        Op8<T> vnreg[VNAT ? NKC : 1];
        Op8<T> vreg[VNAT ? 1 : NVR][4];
        // This thread's 8-element chunks of a K (and bf16 V) tile: element offset
        // within the tile in global memory and in the two LDS layouts.
        constexpr bool FULL = KCH % NTHR == 0;
        int g_off[NKC], k_off[NKC], v_off[NKC];
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = min(tid + n * NTHR, KCH - 1);
            g_off[n] = (c / (D / 8)) * D + (c % (D / 8)) * 8;
            k_off[n] = (c / (D / 8)) * KRS + (c % (D / 8)) * 8;
            v_off[n] = (c / (D / 8)) * VNRS + (c % (D / 8)) * 8;
        }
        auto load_tile = [&](int j) {
            const int key0 = j * KT;
            if (key0 + KT <= T_len) {  // whole tile inside the sequence: no clamping
                const S *kt = kg + static_cast<int64_t>(key0) * D;
                const S *vt = vg + static_cast<int64_t>(key0) * D;
#pragma unroll
                for (int n = 0; n < NKC; ++n) {
                    if (FULL || tid + n * NTHR < KCH) {
                        kreg[n] = op8_load(kt + g_off[n]);
                        if constexpr (VNAT) vnreg[n] = op8_load(vt + g_off[n]);
                    }
                }
            } else {
#pragma unroll
                for (int n = 0; n < NKC; ++n) {
                    const int c = tid + n * NTHR;
                    if (FULL || c < KCH) {
                        const int kk = min(key0 + c / (D / 8), T_len - 1);
                        const int off = (c % (D / 8)) * 8;
                        kreg[n] = op8_load(kg + static_cast<int64_t>(kk) * D + off);
                        if constexpr (VNAT) vnreg[n] = op8_load(vg + static_cast<int64_t>(kk) * D + off);
                    }
                }
            }
            if constexpr (VNAT) return;
#pragma unroll
            for (int n = 0; n < NVR; ++n) {
                const int it = tid + n * NTHR;
                if (it < VRUN) {
                    const int run = it % (KT / 4);
                    const int chunk = it / (KT / 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kk = min(key0 + 4 * run + i, T_len - 1);
                        vreg[n][i] = op8_load(vg + static_cast<int64_t>(kk) * D + chunk * 8);
                    }
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int n = 0; n < NKC; ++n) {
                if (FULL || tid + n * NTHR < KCH) {
                    store_op8(&lds_k[buf][k_off[n]], kreg[n]);
                    if constexpr (VNAT) store_op8(&lds_v[buf][v_off[n]], vnreg[n]);
                }
            }
            if constexpr (VNAT) return;
#pragma unroll
            for (int n = 0; n < NVR; ++n) {
                const int it = tid + n * NTHR;
                if (it < VRUN) {
                    // Consecutive threads take consecutive 4-key runs of one 8-dim
                    // chunk, so a store instruction writes one transposed row.
                    const int run = it % (KT / 4);
                    const int chunk = it / (KT / 4);
                    const int blk = run >> 2, q = run & 3;
                    const int vpos = 32 * (blk >> 1) + 8 * q + 4 * (blk & 1);
#pragma unroll
                    for (int e = 0; e < 8; ++e) store_vt4(&lds_v[buf][(chunk * 8 + e) * VRS + vpos], vreg[n], e);
                }
            }
        };

        float m_run[NB], lsum[NB], csum[NB];
        f32x4 acc_a[NB][DT];
        f32x4 acc_b[NB][HAS_RHO ? DT : 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m_run[nb] = -INFINITY;
            lsum[nb] = 0.f;
            csum[nb] = 0.f;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                acc_a[nb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (HAS_RHO) acc_b[nb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }

        load_tile(0);
        store_tile(0);
        if (TPB > 1 && n_tiles > 1) {
            load_tile(1);
            store_tile(1);
        }

        // One key tile; on the last tile of a persistent item (`last`) the
        // next item's q and rho operands are requested.
        // `nlive`: 16-key blocks of the tile that hold a key of this wavefront's
        // rows (the others are masked for all of them and are skipped: no score
        // or value products, probabilities 0).  Every tile but an item's last
        // (its diagonal tile) passes NKB.
        auto tile_step = [&](const int j, auto last, auto nlive) __attribute__((always_inline)) {
            constexpr int NL = decltype(nlive)::value;  // live 16-key blocks
            constexpr int NUL = (NL + 1) / 2;           // live 32-key slices
            const int buf = j & (NBUF - 1);
            if (j % TPB == 0) __syncthreads();  // tiles j .. j + TPB - 1 are in LDS; the other buffers are free
            const bool more = j + TPB < n_tiles;
            if (more) load_tile(j + TPB);

            const int key0 = j * KT;
            if (key0 <= wpos_last) {
                const bool diag = key0 + KT - 1 > wpos0;
                const S *kt = lds_k[buf];
                const S *vt = lds_v[buf];

                f32x4 sacc[NB][NKB];
                f32x4 racc[NB][HAS_RHO ? NKB : 1];
                // Matrix phases run at raised wave priority so that a wavefront
                // issuing MFMAs gets the issue slots while its SIMD partner is in
                // the VALU-heavy softmax.
                __builtin_amdgcn_s_setprio(1);
                // bf16 with a probe: all K operand reads of the tile go out first,
                // in the order the MFMAs consume them, so the LDS latency is paid
                // once per tile rather than once per 16-key block, and the V
                // operand reads go out before the softmax, whose VALU work then
                // hides their latency (measured: 2-3% faster).  Elsewhere the
                // compiler places the reads (softmax only: the forced order
                // measured 10% slower; fp32: the operands would not fit in
                // registers at once).
                constexpr bool PRE = VNAT && HAS_RHO;
                Op8<T> kop_all[NKB][KS];
#pragma unroll
                for (int kb = 0; kb < NL; ++kb)
#pragma unroll
                    for (int s = 0; s < KS; ++s) kop_all[kb][s] = op8_load(kt + (16 * kb + col) * KRS + 32 * s + 8 * grp);
                if constexpr (PRE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < NL; ++kb) {
                    const Op8<T>(&kop)[KS] = kop_all[kb];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < KS; ++s) a = mma32(kop[s], qop[nb][s], a);
                        sacc[nb][kb] = a;
                        if constexpr (HAS_RHO) {
                            f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s = 0; s < KS; ++s) r = mma32(kop[s], rop[nb][s], r);
                            racc[nb][kb] = r;
                        }
                    }
                }

                __builtin_amdgcn_s_setprio(0);
                // V operand reads.
                auto load_vop = [&](int u, int t) {
                    if constexpr (VNAT) {
                        // Lane col of group grp names key 32u + 4grp + col/4 (and
                        // that key + 16) at dims 16t + 4(col%4) .. +3; the transposed
                        // read returns to lane col dim 16t + col of the 4 keys named
                        // by lanes col/4, col/4 + 4, col/4 + 8, col/4 + 12, i.e. keys
                        // 32u + 4grp + 0..3: the k-slots of this lane group.
                        const S *a = vt + (32 * u + 4 * grp + (col >> 2)) * VNRS + 16 * t + 4 * (col & 3);
                        return op8_load_tr(a, a + 16 * VNRS);
                    } else {
                        return op8_load(vt + (16 * t + col) * VRS + 32 * u + 8 * grp);
                    }
                };
                constexpr bool VPRE = PRE;
                Op8<T> vop_all[VPRE ? NU : 1][VPRE ? DT : 1];
                if constexpr (VPRE) {
#pragma unroll
                    for (int u = 0; u < NUL; ++u)
#pragma unroll
                        for (int t = 0; t < DT; ++t) vop_all[u][t] = load_vop(u, t);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (decltype(last)::value) {
                    load_rows(next, wave, col, grp, nq, nr);
                    __builtin_amdgcn_sched_barrier(0);
                }
                Op8<T> pop[NB][NU];
                Op8<T> prop[NB][HAS_RHO ? NU : 1];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    // Raw scores; the scale is folded into the exponent below.
                    float x[NKB * 4];
#pragma unroll
                    for (int e = 0; e < NKB * 4; ++e) x[e] = e < NL * 4 ? sacc[nb][e >> 2][e & 3] : -INFINITY;
                    if (diag) {  // wave-uniform: only tiles that cross the diagonal
                        const int rel = pos[nb] - key0 - 4 * grp;  // key > pos <=> offset > rel
#pragma unroll
                        for (int e = 0; e < NL * 4; ++e)
                            if (16 * (e >> 2) + (e & 3) > rel) x[e] = -INFINITY;
                    }
                    float mt = -INFINITY;
#pragma unroll
                    for (int e = 0; e < NL * 4; ++e) mt = fmaxf(mt, x[e]);
                    mt *= p.scale_log2;  // this lane's max; the row max needs 4 lanes
                    // The running max only moves when some row's max grows by more
                    // than kRescaleSlack (log2 units), so P stays below 2^slack and
                    // the rescale of l, c, A, B is rare.  Testing each lane's own
                    // max is enough to decide (wave-uniformly); the cross-lane row
                    // max is only formed when a rescale happens.
                    if (wave_any(mt > m_run[nb] + kRescaleSlack)) {
                        mt = row_group_max(mt);
                        const float m_new = fmaxf(m_run[nb], mt);
                        const float alpha = fast_exp2(m_run[nb] - m_new);
                        m_run[nb] = m_new;
                        lsum[nb] *= alpha;
                        if constexpr (HAS_RHO) csum[nb] *= alpha;
#pragma unroll
                        for (int t = 0; t < DT; ++t) {
                            acc_a[nb][t] *= alpha;
                            if constexpr (HAS_RHO) acc_b[nb][t] *= alpha;
                        }
                    }
                    const float neg_m = -m_run[nb];
                    float pr[NKB * 4];
#pragma unroll
                    for (int e = 0; e < NUL * 8; ++e) {
                        x[e] = e < NL * 4 ? fast_exp2(fmaf(x[e], p.scale_log2, neg_m)) : 0.f;
                        if constexpr (HAS_RHO) pr[e] = e < NL * 4 ? x[e] * racc[nb][e >> 2][e & 3] : 0.f;
                    }
                    // Row sums over the rounded operands (see op8_sum_acc).
#pragma unroll
                    for (int u = 0; u < NUL; ++u) {
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = x[8 * u + e];
                        pop[nb][u] = op8_pack(w, T{});
                        lsum[nb] = op8_sum_acc(pop[nb][u], lsum[nb]);
                        if constexpr (HAS_RHO) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) w[e] = pr[8 * u + e];
                            prop[nb][u] = op8_pack(w, T{});
                            csum[nb] = op8_sum_acc(prop[nb][u], csum[nb]);
                        }
                    }
                }

                if constexpr (PRE) __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int u = 0; u < NUL; ++u) {
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        const Op8<T> vop = VPRE ? vop_all[VPRE ? u : 0][VPRE ? t : 0] : load_vop(u, t);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            acc_a[nb][t] = mma32(vop, pop[nb][u], acc_a[nb][t]);
                            if constexpr (HAS_RHO) acc_b[nb][t] = mma32(vop, prop[nb][u], acc_b[nb][t]);
                        }
                    }
                }
            } else if constexpr (decltype(last)::value) {
                load_rows(next, wave, col, grp, nq, nr);
            }

            __builtin_amdgcn_s_setprio(0);
            if (more) store_tile((j + TPB) & (NBUF - 1));
        };
        using AllBlocks = std::integral_constant<int, NKB>;
        if constexpr (PERSIST) {
            for (int j = 0; j < n_tiles - 1; ++j) tile_step(j, std::false_type{}, AllBlocks{});
            // The last tile holds the diagonal: this wavefront's rows reach
            // (wpos_last - key0) / 16 + 1 of its 16-key blocks (wave-uniform).
            const int jl = n_tiles - 1;
            const int nl = min(NKB, max(1, (wpos_last - jl * KT) / 16 + 1));
            static_assert(!PERSIST || NKB == 4, "the last-tile dispatch covers 4 blocks");
            if (nl == 1) tile_step(jl, std::true_type{}, std::integral_constant<int, 1>{});
            else if (nl == 2) tile_step(jl, std::true_type{}, std::integral_constant<int, 2>{});
            else if (nl == 3) tile_step(jl, std::true_type{}, std::integral_constant<int, 3>{});
            else tile_step(jl, std::true_type{}, AllBlocks{});
        } else {
            for (int j = 0; j < n_tiles; ++j) tile_step(j, std::false_type{}, AllBlocks{});
        }

        // Epilogue: acc[nb][t][i] is head-dim 16*t + 4*grp + i of this lane's row.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float l = row_group_sum(lsum[nb]);
            const float c = HAS_RHO ? row_group_sum(csum[nb]) : 0.f;
            if (pos[nb] < T_len) {
                const float inv = 1.f / l;
                const float cbar = c * inv;
                S *o = static_cast<S *>(p.out) + qoff[nb];
                S *osa_out = p.out_sa ? static_cast<S *>(p.out_sa) + qoff[nb] : nullptr;
                if constexpr (VNAT) {
                    // 16-byte stores: the lanes of 16-lane rows 2k and 2k + 1 (same
                    // column, so same output row) swap halves with
                    // v_permlane16_swap, so that each lane holds 8 consecutive head
                    // dims: rows 0 and 2 take the even 16-dim tiles, rows 1 and 3
                    // the odd ones.
                    auto pack_tile = [&](int t, bool sa, uint32_t (&w)[2]) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float osa = acc_a[nb][t][i] * inv;
                            if constexpr (HAS_RHO) {
                                const float corr = acc_b[nb][t][i] * inv - cbar * osa;
                                y[i] = sa ? osa : osa - corr;
                            } else {
                                y[i] = osa;
                            }
                        }
                        w[0] = pack2_bf16(y[0], y[1]);
                        w[1] = pack2_bf16(y[2], y[3]);
                    };
                    const int dim0 = 8 * (grp >> 1) + 16 * (grp & 1);
#pragma unroll
                    for (int t = 0; t < DT; t += 2) {
                        uint32_t e[2], f[2];
                        pack_tile(t, false, e);
                        pack_tile(t + 1, false, f);
                        const auto w0 = __builtin_amdgcn_permlane16_swap(e[0], f[0], false, false);
                        const auto w1 = __builtin_amdgcn_permlane16_swap(e[1], f[1], false, false);
                        const u32x4 v = u32x4{w0[0], w1[0], w0[1], w1[1]};
                        u32x4 *dst = reinterpret_cast<u32x4 *>(o + 16 * t + dim0);
                        // Softmax-only output as streaming stores (measured 1.5%
                        // faster there, slower for the probe kernel).
                        if constexpr (HAS_RHO) *dst = v;
                        else __builtin_nontemporal_store(v, dst);
                        if (osa_out) {
                            pack_tile(t, true, e);
                            pack_tile(t + 1, true, f);
                            const auto s0 = __builtin_amdgcn_permlane16_swap(e[0], f[0], false, false);
                            const auto s1 = __builtin_amdgcn_permlane16_swap(e[1], f[1], false, false);
                            *reinterpret_cast<u32x4 *>(osa_out + 16 * t + dim0) = u32x4{s0[0], s1[0], s0[1], s1[1]};
                        }
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        float y[4], ysa[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float osa = acc_a[nb][t][i] * inv;
                            ysa[i] = osa;
                            if constexpr (HAS_RHO) {
                                const float corr = acc_b[nb][t][i] * inv - cbar * osa;
                                y[i] = osa - corr;
                            } else {
                                y[i] = osa;
                            }
                        }
                        store4(o + 16 * t + 4 * grp, y);
                        if (osa_out) store4(osa_out + 16 * t + 4 * grp, ysa);
                    }
                }
                // Training forward: the row's log2-sum-exp (P = 2^(s log2e - m)
                // summed to l, so log2 sum_j 2^(s_j log2e) = m + log2 l) and rbar.
                if (p.lse != nullptr && grp == 0) {
                    const int64_t row = qoff[nb] / D;
                    p.lse[row] = m_run[nb] + log2f(l);
                    if (p.rbar) p.rbar[row] = cbar;
                }
            }
        }
    };  // run_item

    if constexpr (PERSIST) {
        // The grid is then a multiple of 8 workgroups, fewer than the items:
        // workgroup (xcd, c), c < ncu, takes in round r the slot
        // r*ncu + c (r even) or r*ncu + ncu-1-c (r odd) of its XCD's item list,
        // so the long and short query blocks of a unit pair up (every slot is
        // taken once: within a round c -> slot is a bijection).  A grid of
        // one workgroup per item takes item blockIdx.x.
        const int n_items = n_units * p.n_qblk;
        const bool persist = static_cast<int>(gridDim.x) < n_items;
        const int xcd = blockIdx.x % kXcds, c = blockIdx.x / kXcds, ncu = gridDim.x / kXcds;
        auto item_at = [&](int r) {
            return persist ? xcd + kXcds * (r * ncu + ((r & 1) ? ncu - 1 - c : c))
                           : (r == 0 ? static_cast<int>(blockIdx.x) : n_items);
        };
        const int lane0 = threadIdx.x & (kWave - 1);
        int id = item_at(0);
        if (id < n_items) load_rows(id, threadIdx.x / kWave, lane0 & 15, lane0 >> 4, nq, nr);
        for (int r = 0; id < n_items; ++r) {  // later rounds only hold larger slots
            const int next = item_at(r + 1);
            // With no next item the last tile requests this item's rows again
            // (always a valid address; unused).
            run_item(id, next < n_items ? next : id);
            // The next item's first tiles overwrite LDS buffers 0 and 1, so all
            // waves meet here.  Every LDS read of this item has completed (its
            // data fed the value products before the epilogue), so the barrier
            // needs no wait: this item's output stores and the next item's
            // q / rho loads stay in flight (__syncthreads() would wait for
            // them).  The empty asm statements keep the compiler from moving
            // memory accesses across the barrier.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            id = next;
        }
    } else {
        run_item(blockIdx.x, blockIdx.x);
    }
}

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

template <class T, int D, int G, bool R>
hipError_t launch_prefill_r(const PrefillParams &p, hipStream_t stream) {
    int64_t blocks = static_cast<int64_t>(p.B) * p.Hkv * p.n_qblk;
    if constexpr (std::is_same<T, BF16>::value && R) {
        // Persistent grid: one workgroup per CU, a multiple of the 8 XCDs.
        const int64_t grid = device_cus() / kXcds * kXcds;
        if (grid > 0 && blocks > grid) blocks = grid;
    }
    hipLaunchKernelGGL((prefill_kernel<T, D, G, R>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kPrefillWaves * kWave), 0, stream, p);
    return hipGetLastError();
}

template <class T, int D, int G>
hipError_t launch_prefill_g(const PrefillParams &p, bool has_rho, hipStream_t stream) {
    return has_rho ? launch_prefill_r<T, D, G, true>(p, stream) : launch_prefill_r<T, D, G, false>(p, stream);
}

template <class T, int D>
hipError_t launch_prefill_d(const PrefillParams &p, int G, bool has_rho, hipStream_t stream) {
    switch (G) {
    case 1: return launch_prefill_g<T, D, 1>(p, has_rho, stream);
    case 2: return launch_prefill_g<T, D, 2>(p, has_rho, stream);
    case 4: return launch_prefill_g<T, D, 4>(p, has_rho, stream);
    case 8: return launch_prefill_g<T, D, 8>(p, has_rho, stream);
    default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t launch_prefill_t(const PrefillParams &p, int D, int G, bool has_rho, hipStream_t stream) {
    switch (D) {
    case 64: return launch_prefill_d<T, 64>(p, G, has_rho, stream);
    case 128: return launch_prefill_d<T, 128>(p, G, has_rho, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int prefill_block_positions(bool /*bf16*/, int G) { return 16 * kColTiles / G * kPrefillWaves; }

hipError_t launch_prefill(const PrefillParams &p, bool bf16, int D, int G, bool has_rho, hipStream_t stream) {
    return bf16 ? launch_prefill_t<BF16>(p, D, G, has_rho, stream)
                : launch_prefill_t<F32>(p, D, G, has_rho, stream);
}

}  // namespace plx
