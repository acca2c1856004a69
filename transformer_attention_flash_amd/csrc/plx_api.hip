// plx_api.hip -- the extern "C" entry points of libparallax.so: argument
// checks (host only, before any HIP call), split and workspace policy, and the
// kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/parallax.h"
#include "plx_kernels.h"

// Scratch of parallax_fwd_decode_noalloc: the per-chunk partial results of a
// split decode, for callers that cannot allocate.  Each device holds its own
// copy from the first call on it until the process ends.  In host code this
// name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress (noalloc_scratch below) and is the only form passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[PLX_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t kMaxKeysPerSplit = 1 << 20;
constexpr int64_t kMaxGrid = (int64_t{1} << 31) - 1;

bool supported_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }
bool valid_scale(float s) { return isfinite(s) && s > 0.f; }
size_t elem_bytes(plx_dtype_t t) { return t == PLX_DTYPE_BF16 ? 2 : 4; }

// The kernels read and write 8-element vectors: every tensor must start on a
// 16-byte boundary.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// Shape checks shared by both entry points.
plx_status_t check_heads(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, float scale, plx_dtype_t dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || d < 1) return PLX_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv != 0) return PLX_ERR_INVALID_ARGUMENT;
    if (!valid_scale(scale)) return PLX_ERR_INVALID_ARGUMENT;
    if (dtype != PLX_DTYPE_BF16 && dtype != PLX_DTYPE_F32) return PLX_ERR_UNSUPPORTED;
    if (!supported_dim(d) || !supported_group(Hq / Hkv)) return PLX_ERR_UNSUPPORTED;
    return PLX_OK;
}

// Keys per chunk when the caller leaves it to the library.  A chunk is one
// workgroup of up to 8 wavefronts (one per 128 keys) that merge their states
// in LDS, so large chunks are cheap.  Chunks are as large as possible -- one
// per sequence, so no merge kernel runs -- unless that launches fewer than
// 512 workgroups (2 per CU), in which case they are halved until it does or
// reach 256 keys.  Measured on the decode workloads: one chunk per sequence
// is best for 4096 keys x 64 sequences and for a ragged batch of 2048
// sequences (8 chunks per sequence there cost 1.5x), and within 1% for 256
// sequences of 32768 keys.  Contexts of up to 256 keys use one 256-key chunk
// (two wavefronts), which measured faster than one wavefront at 128 keys.
int32_t auto_keys_per_split(int64_t units, int64_t max_ctx) {
    if (max_ctx <= 256) return 256;
    int32_t ks = 256;
    while (ks < max_ctx && ks < kMaxKeysPerSplit) ks *= 2;
    while (ks > 256 && units * ((max_ctx + ks - 1) / ks) < 512) ks /= 2;
    return ks;
}

struct DecodePlan {
    int32_t keys_per_split;
    int32_t n_split;
    size_t stats_bytes;  // offset of the vector block
    size_t bytes;        // total workspace
};

plx_status_t plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t max_ctx, plx_dtype_t dtype,
                         int32_t keys_per_split, DecodePlan *plan) {
    plx_status_t st = check_heads(B, Hq, Hkv, d, 1.f, dtype);
    if (st != PLX_OK) return st;
    if (max_ctx < 0) return PLX_ERR_INVALID_ARGUMENT;
    if (keys_per_split != 0 &&
        (keys_per_split < 32 || keys_per_split > kMaxKeysPerSplit || keys_per_split % 32 != 0))
        return PLX_ERR_INVALID_ARGUMENT;
    const int64_t units = static_cast<int64_t>(B) * Hkv;
    const int32_t ks = keys_per_split ? keys_per_split : auto_keys_per_split(units, max_ctx);
    int64_t n_split = (max_ctx + ks - 1) / ks;
    if (n_split < 1) n_split = 1;
    if (units * n_split > kMaxGrid || static_cast<int64_t>(B) * Hq > kMaxGrid) return PLX_ERR_UNSUPPORTED;
    plan->keys_per_split = ks;
    plan->n_split = static_cast<int32_t>(n_split);
    if (n_split == 1) {
        plan->stats_bytes = 0;
        plan->bytes = 0;
    } else {
        const size_t slots = static_cast<size_t>(B) * Hq * static_cast<size_t>(n_split);
        plan->stats_bytes = (slots * 3 * sizeof(float) + 255) & ~size_t{255};
        plan->bytes = plan->stats_bytes + slots * 2 * static_cast<size_t>(d) * sizeof(float);
    }
    return PLX_OK;
}

// Causal prefill forward; the training variant also keeps (out_sa, lse, rbar).
plx_status_t prefill_impl(const void *q, const void *k, const void *v, const void *rho, void *out, void *out_sa,
                          float *lse, float *rbar, int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d,
                          float softmax_scale, plx_dtype_t dtype, hipStream_t stream) {
    if (!q || !k || !v || !out) return PLX_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(rho) || !aligned16(out) ||
        !aligned16(out_sa) || !aligned16(lse) || !aligned16(rbar))
        return PLX_ERR_INVALID_ARGUMENT;
    if (T < 1) return PLX_ERR_INVALID_ARGUMENT;
    plx_status_t st = check_heads(B, Hq, Hkv, d, softmax_scale, dtype);
    if (st != PLX_OK) return st;
    const int G = Hq / Hkv;
    const bool bf16 = dtype == PLX_DTYPE_BF16;
    const int bq = plx::prefill_block_positions(bf16, G);
    const int64_t n_qblk = (static_cast<int64_t>(T) + bq - 1) / bq;
    if (static_cast<int64_t>(B) * Hkv * n_qblk > kMaxGrid) return PLX_ERR_UNSUPPORTED;

    const size_t es = elem_bytes(dtype);
    const size_t q_bytes = static_cast<size_t>(B) * Hq * T * d * es;
    const size_t kv_bytes = static_cast<size_t>(B) * Hkv * T * d * es;
    const size_t st_bytes = static_cast<size_t>(B) * Hq * T * sizeof(float);
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}, {rho, q_bytes}};
    const Span outs[] = {{out, q_bytes}, {out_sa, q_bytes}, {lse, st_bytes}, {rbar, st_bytes}};
    for (const Span &o : outs) {
        for (const Span &x : ins)
            if (overlaps(o.p, o.n, x.p, x.n)) return PLX_ERR_INVALID_ARGUMENT;
        for (const Span &x : outs)
            if (&x != &o && overlaps(o.p, o.n, x.p, x.n)) return PLX_ERR_INVALID_ARGUMENT;
    }

    plx::PrefillParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.rho = rho;
    p.out = out;
    p.out_sa = out_sa;
    p.lse = lse;
    p.rbar = rbar;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.T = T;
    p.n_qblk = static_cast<int32_t>(n_qblk);
    p.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
    const hipError_t e = plx::launch_prefill(p, bf16, d, G, rho != nullptr, stream);
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

// Device address of `scratch` on the device that runs `stream` (its own copy
// per device), resolved once per device with that device current.  The only
// HIP calls are the device queries and, on a device's first use,
// hipGetSymbolAddress; nothing is allocated here.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

plx_status_t noalloc_scratch(hipStream_t stream, void **ptr) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return PLX_ERR_HIP;
    dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return PLX_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return PLX_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return PLX_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return PLX_ERR_HIP;
        if (e != hipSuccess || p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return PLX_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PLX_OK;
}

// Decode; with use_scratch the partials go to the library's static scratch
// instead of the caller's workspace (workspace / workspace_bytes unused).
plx_status_t decode_impl(const void *q, const void *rho, const void *k_cache, const void *v_cache,
                         const int64_t *cu_seqlens, int64_t max_ctx, void *out, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t d, float softmax_scale, plx_dtype_t dtype, int32_t keys_per_split, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, bool use_scratch = false) {
    if (!q || !out) return PLX_ERR_INVALID_ARGUMENT;
    // With max_ctx == 0 every sequence is empty and no key is read, so an
    // empty cache may come without storage.
    if (max_ctx != 0 && (!k_cache || !v_cache)) return PLX_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(workspace) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0)
        return PLX_ERR_INVALID_ARGUMENT;
    plx_status_t st = check_heads(B, Hq, Hkv, d, softmax_scale, dtype);
    if (st != PLX_OK) return st;
    DecodePlan plan;
    st = plan_decode(B, Hq, Hkv, d, max_ctx, dtype, keys_per_split, &plan);
    if (st != PLX_OK) return st;
    if (use_scratch) {
        if (plan.bytes > PLX_DECODE_NOALLOC_SCRATCH_BYTES) return PLX_ERR_WORKSPACE_TOO_SMALL;
        workspace = nullptr;
        workspace_bytes = 0;
    } else if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) {
        return PLX_ERR_WORKSPACE_TOO_SMALL;
    }

    const size_t es = elem_bytes(dtype);
    const size_t q_bytes = static_cast<size_t>(B) * Hq * d * es;
    if (overlaps(out, q_bytes, q, q_bytes) || overlaps(out, q_bytes, rho, q_bytes) ||
        overlaps(out, q_bytes, workspace, plan.bytes))
        return PLX_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens) {
        const size_t kv_bytes = static_cast<size_t>(B) * Hkv * static_cast<size_t>(max_ctx) * d * es;
        if (overlaps(out, q_bytes, k_cache, kv_bytes) || overlaps(out, q_bytes, v_cache, kv_bytes))
            return PLX_ERR_INVALID_ARGUMENT;
    }

    // Every argument check is done; only now may HIP be called.
    if (use_scratch && plan.bytes > 0) {
        st = noalloc_scratch(stream, &workspace);
        if (st != PLX_OK) return st;
    }

    plx::DecodeParams p;
    p.q = q;
    p.rho = rho;
    p.k = k_cache;
    p.v = v_cache;
    p.cu = cu_seqlens;
    p.max_ctx = max_ctx;
    p.out = out;
    p.ws_stats = plan.bytes ? static_cast<float *>(workspace) : nullptr;
    p.ws_vec = plan.bytes ? reinterpret_cast<float *>(static_cast<char *>(workspace) + plan.stats_bytes) : nullptr;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.keys_per_split = plan.keys_per_split;
    p.n_split = plan.n_split;
    p.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
    const hipError_t e = plx::launch_decode(p, dtype == PLX_DTYPE_BF16, d, Hq / Hkv, stream);
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

}  // namespace

extern "C" {

plx_status_t parallax_fwd_prefill(const void *q, const void *k, const void *v, const void *rho, void *out,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d,
                                  float softmax_scale, plx_dtype_t dtype, hipStream_t stream) {
    return prefill_impl(q, k, v, rho, out, nullptr, nullptr, nullptr, B, Hq, Hkv, T, d, softmax_scale, dtype,
                        stream);
}

plx_status_t parallax_fwd_prefill_train(const void *q, const void *k, const void *v, const void *rho, void *out,
                                        void *out_sa, float *lse, float *rbar, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t T, int32_t d, float softmax_scale,
                                        plx_dtype_t dtype, hipStream_t stream) {
    if (!lse) return PLX_ERR_INVALID_ARGUMENT;
    if ((rho == nullptr) != (out_sa == nullptr) || (rho == nullptr) != (rbar == nullptr))
        return PLX_ERR_INVALID_ARGUMENT;
    if (dtype != PLX_DTYPE_BF16) return PLX_ERR_UNSUPPORTED;
    return prefill_impl(q, k, v, rho, out, out_sa, lse, rbar, B, Hq, Hkv, T, d, softmax_scale, dtype, stream);
}

size_t parallax_bwd_prefill_workspace_size(int32_t B, int32_t Hq, int32_t T) {
    if (B < 1 || Hq < 1 || T < 1) return ~size_t{0};
    return static_cast<size_t>(B) * Hq * T * 4 * sizeof(float);
}

plx_status_t parallax_bwd_prefill(const void *q, const void *k, const void *v, const void *rho, const void *out,
                                  const void *out_sa, const float *lse, const float *rbar, const void *dout,
                                  void *dq, void *dk, void *dv, void *drho, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t T, int32_t d, float softmax_scale, plx_dtype_t dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return PLX_ERR_INVALID_ARGUMENT;
    const bool has_rho = rho != nullptr;
    if (has_rho != (out_sa != nullptr) || has_rho != (rbar != nullptr) || has_rho != (drho != nullptr))
        return PLX_ERR_INVALID_ARGUMENT;
    const void *ptrs[] = {q, k, v, rho, out, out_sa, lse, rbar, dout, dq, dk, dv, drho, workspace};
    for (const void *x : ptrs)
        if (!aligned16(x)) return PLX_ERR_INVALID_ARGUMENT;
    if (T < 1) return PLX_ERR_INVALID_ARGUMENT;
    plx_status_t st = check_heads(B, Hq, Hkv, d, softmax_scale, dtype);
    if (st != PLX_OK) return st;
    if (dtype != PLX_DTYPE_BF16) return PLX_ERR_UNSUPPORTED;
    const size_t need = parallax_bwd_prefill_workspace_size(B, Hq, T);
    if (workspace_bytes < need) return PLX_ERR_WORKSPACE_TOO_SMALL;
    const int G = Hq / Hkv;
    // The kernels index the rows of a KV group (position x G + head) in 32 bits.
    if (static_cast<int64_t>(T) * G >= (int64_t{1} << 31)) return PLX_ERR_UNSUPPORTED;
    const int bq = plx::backward_q_block_positions(G);
    const int kb = plx::backward_k_block_keys();
    const int64_t n_qblk = (static_cast<int64_t>(T) + bq - 1) / bq;
    const int64_t n_kblk = (static_cast<int64_t>(T) + kb - 1) / kb;
    const int64_t units = static_cast<int64_t>(B) * Hkv;
    const int64_t rows = static_cast<int64_t>(B) * Hq * T;
    if (units * n_qblk > kMaxGrid || units * n_kblk > kMaxGrid || (rows + 15) / 16 > kMaxGrid)
        return PLX_ERR_UNSUPPORTED;

    // No output may overlap an input, another output or the workspace.
    const size_t qb = static_cast<size_t>(rows) * d * 2;
    const size_t kvb = static_cast<size_t>(B) * Hkv * T * d * 2;
    const size_t sb = static_cast<size_t>(rows) * sizeof(float);
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{q, qb}, {k, kvb}, {v, kvb}, {rho, qb}, {out, qb}, {out_sa, qb}, {lse, sb}, {rbar, sb},
                        {dout, qb}, {workspace, need}};
    const Span outs[] = {{dq, qb}, {dk, kvb}, {dv, kvb}, {drho, qb}};
    for (const Span &o : outs) {
        for (const Span &x : ins)
            if (overlaps(o.p, o.n, x.p, x.n)) return PLX_ERR_INVALID_ARGUMENT;
        for (const Span &x : outs)
            if (&x != &o && overlaps(o.p, o.n, x.p, x.n)) return PLX_ERR_INVALID_ARGUMENT;
    }

    plx::BackwardParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.rho = rho;
    p.out = out;
    p.out_sa = out_sa;
    p.lse = lse;
    p.rbar = rbar;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.drho = drho;
    p.rowst = static_cast<float4 *>(workspace);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.T = T;
    p.n_qblk = static_cast<int32_t>(n_qblk);
    p.n_kblk = static_cast<int32_t>(n_kblk);
    p.scale = softmax_scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
    const hipError_t e = plx::launch_backward(p, d, G, stream);
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t parallax_qkvr_projection(const void *x, const void *w, void *q, void *k, void *v, void *rho,
                                      int32_t B, int32_t T, int32_t d_model, int32_t Hq, int32_t Hkv, int32_t d,
                                      plx_dtype_t dtype, hipStream_t stream) {
    if (!x || !w || !q || !k || !v || !rho) return PLX_ERR_INVALID_ARGUMENT;
    const void *ptrs[] = {x, w, q, k, v, rho};
    for (const void *ptr : ptrs)
        if (!aligned16(ptr)) return PLX_ERR_INVALID_ARGUMENT;
    if (B < 1 || T < 1 || d_model < 1 || Hq < 1 || Hkv < 1 || d < 1) return PLX_ERR_INVALID_ARGUMENT;
    if (dtype != PLX_DTYPE_BF16 && dtype != PLX_DTYPE_F32) return PLX_ERR_UNSUPPORTED;
    if (dtype != PLX_DTYPE_BF16 || !supported_dim(d) || d_model % plx::projection_step() != 0)
        return PLX_ERR_UNSUPPORTED;
    const int64_t n_tokens = static_cast<int64_t>(B) * T;
    const int64_t features = (2 * static_cast<int64_t>(Hq) + 2 * Hkv) * d;
    const int64_t n_fblk = (features + plx::projection_block_features() - 1) / plx::projection_block_features();
    const int64_t n_tblk = (n_tokens + plx::projection_block_tokens() - 1) / plx::projection_block_tokens();
    if (n_fblk * n_tblk > kMaxGrid || features > (int64_t{1} << 30)) return PLX_ERR_UNSUPPORTED;

    const size_t xb = static_cast<size_t>(n_tokens) * d_model * 2;
    const size_t wb = static_cast<size_t>(features) * d_model * 2;
    const size_t qb = static_cast<size_t>(n_tokens) * Hq * d * 2;
    const size_t kb = static_cast<size_t>(n_tokens) * Hkv * d * 2;
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{x, xb}, {w, wb}};
    const Span outs[] = {{q, qb}, {k, kb}, {v, kb}, {rho, qb}};
    for (const Span &o : outs) {
        for (const Span &in : ins)
            if (overlaps(o.p, o.n, in.p, in.n)) return PLX_ERR_INVALID_ARGUMENT;
        for (const Span &other : outs)
            if (&other != &o && overlaps(o.p, o.n, other.p, other.n)) return PLX_ERR_INVALID_ARGUMENT;
    }

    plx::ProjectionParams p;
    p.x = x;
    p.w = w;
    p.q = q;
    p.k = k;
    p.v = v;
    p.rho = rho;
    p.n_tokens = n_tokens;
    p.T = T;
    p.d_model = d_model;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.nq = Hq * d;
    p.nkv = Hkv * d;
    p.n_fblk = static_cast<int32_t>(n_fblk);
    p.n_tblk = static_cast<int32_t>(n_tblk);
    const hipError_t e = plx::launch_projection(p, stream);
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

size_t parallax_fwd_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t max_ctx,
                                          plx_dtype_t dtype) {
    return parallax_fwd_decode_chunked_workspace_size(B, Hq, Hkv, d, max_ctx, dtype, 0);
}

size_t parallax_fwd_decode_chunked_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t max_ctx,
                                                  plx_dtype_t dtype, int32_t keys_per_split) {
    DecodePlan plan;
    if (plan_decode(B, Hq, Hkv, d, max_ctx, dtype, keys_per_split, &plan) != PLX_OK) return ~size_t{0};
    return plan.bytes;
}

int32_t parallax_fwd_decode_auto_split(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t max_ctx) {
    DecodePlan plan;
    const plx_status_t st = plan_decode(B, Hq, Hkv, d, max_ctx, PLX_DTYPE_BF16, 0, &plan);
    return st == PLX_OK ? plan.keys_per_split : -static_cast<int32_t>(st);
}

plx_status_t parallax_fwd_decode(const void *q, const void *rho, const void *k_cache, const void *v_cache,
                                 const int64_t *cu_seqlens, int64_t max_ctx, void *out, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t d, float softmax_scale, plx_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(q, rho, k_cache, v_cache, cu_seqlens, max_ctx, out, B, Hq, Hkv, d, softmax_scale, dtype, 0,
                       workspace, workspace_bytes, stream);
}

plx_status_t parallax_fwd_decode_chunked(const void *q, const void *rho, const void *k_cache, const void *v_cache,
                                         const int64_t *cu_seqlens, int64_t max_ctx, void *out, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d, float softmax_scale, plx_dtype_t dtype,
                                         int32_t keys_per_split, void *workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    return decode_impl(q, rho, k_cache, v_cache, cu_seqlens, max_ctx, out, B, Hq, Hkv, d, softmax_scale, dtype,
                       keys_per_split, workspace, workspace_bytes, stream);
}

plx_status_t parallax_fwd_decode_noalloc(const void *q, const void *rho, const void *k_cache, const void *v_cache,
                                         const int64_t *cu_seqlens, int64_t max_ctx, void *out, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d, float softmax_scale, plx_dtype_t dtype,
                                         hipStream_t stream) {
    return decode_impl(q, rho, k_cache, v_cache, cu_seqlens, max_ctx, out, B, Hq, Hkv, d, softmax_scale, dtype, 0,
                       nullptr, 0, stream, true);
}

const char *parallax_status_string(plx_status_t s) {
    switch (s) {
    case PLX_OK: return "ok";
    case PLX_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PLX_ERR_UNSUPPORTED: return "unsupported configuration";
    case PLX_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PLX_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

}  // extern "C"
