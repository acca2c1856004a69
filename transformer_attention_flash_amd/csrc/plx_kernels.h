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
    int32_t B, Hq, Hkv, T;
    int32_t n_qblk;     // query blocks per (b, kv head)
    float scale_log2;
};

// Both return the first launch error (hipSuccess when everything queued).
hipError_t launch_decode(const DecodeParams &p, bool bf16, int D, int G, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, bool bf16, int D, int G, bool has_rho,
                          hipStream_t stream);

// Query positions one prefill workgroup covers for group size G.
int prefill_block_positions(bool bf16, int G);

}  // namespace plx
