// plx_kernels.h -- kernel parameter blocks and launchers of libparallax
// (internal; the public interface is include/parallax.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

struct DecodeParams {
    const void *q;      // [B, Hq, D]
    const void *rho;    // [B, Hq, D] or null (zero probe)
    const void *k;      // cache, see seq_view
    const void *v;
    const int64_t *cu;  // device [B + 1] token offsets or null (contiguous)
    int64_t max_ctx;
    void *out;          // [B, Hq, D]
    float *ws_stats;    // [B*Hq, n_split, 3]: m, l, c of each chunk
    float *ws_vec;      // [B*Hq, n_split, 2, D]: A, B of each chunk
    int32_t B, Hq, Hkv;
    int32_t keys_per_split;
    int32_t n_split;    // chunks per sequence = ceil(max_ctx / keys_per_split)
    float scale_log2;   // softmax scale * log2(e)
};

struct PrefillParams {
    const void *q;      // [B, Hq, T, D]
    const void *k;      // [B, Hkv, T, D]
    const void *v;
    const void *rho;    // [B, Hq, T, D] (unused by the softmax-only kernel)
    void *out;          // [B, Hq, T, D]
    // Training forward only (all null otherwise): what the backward needs.
    void *out_sa;       // [B, Hq, T, D] softmax-attention part A/l (null: not kept)
    float *lse;         // [B, Hq, T] log2 of sum_j 2^(s_ij * log2 e), s = scale * q.k
    float *rbar;        // [B, Hq, T] c/l = sum_j p_ij (rho_i . k_j)
    int32_t B, Hq, Hkv, T;
    int32_t n_qblk;     // query blocks per (b, kv head)
    float scale_log2;
};

struct BackwardParams {
    const void *q, *k, *v, *rho;   // forward inputs (rho null: softmax only)
    const void *out, *out_sa;      // forward outputs (out_sa null when rho is)
    const float *lse, *rbar;       // forward row statistics
    const void *dout;              // [B, Hq, T, D] upstream gradient
    void *dq, *dk, *dv, *drho;     // gradients, shaped like q, k, v, rho
    float4 *rowst;                 // workspace [B, Hq, T]: (lse, 1 + rbar, G, -Dsum)
    int32_t B, Hq, Hkv, T;
    int32_t n_qblk;                // dq kernel: query blocks per (b, kv head)
    int32_t n_kblk;                // dk/dv kernel: key blocks per (b, kv head)
    float scale;                   // softmax scale
    float scale_log2;              // softmax scale * log2(e)
};

struct ProjectionParams {
    const void *x;                 // [n_tokens, d_model] (tokens = B x T, row-major)
    const void *w;                 // [(2 Hq + 2 Hkv) d, d_model]: q, k, v, probe rows
    void *q, *k, *v, *rho;         // [B, Hq | Hkv, T, d]
    int64_t n_tokens;
    int32_t T, d_model, Hq, Hkv, d;
    int32_t nq, nkv;               // Hq d, Hkv d
    int32_t n_fblk, n_tblk;        // feature and token blocks
};

// Compute units of the current device (cached per device; 0 if the query
// fails).  The persistent kernels launch one workgroup per CU.
int device_cus();

// Both return the first launch error (hipSuccess when everything queued).
hipError_t launch_decode(const DecodeParams &p, bool bf16, int D, int G, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, bool bf16, int D, int G, bool has_rho,
                          hipStream_t stream);

// Query positions one prefill workgroup covers for group size G.
int prefill_block_positions(bool bf16, int G);

// Prefill backward (bf16): row statistics, then dq/drho and dk/dv.
hipError_t launch_backward(const BackwardParams &p, int D, int G, hipStream_t stream);
int backward_q_block_positions(int G);
int backward_k_block_keys();

// Fused q/k/v/probe projection (bf16).
hipError_t launch_projection(const ProjectionParams &p, hipStream_t stream);
int projection_block_features();
int projection_block_tokens();
int projection_step();

}  // namespace plx
