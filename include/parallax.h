/*
 * parallax.h -- C ABI of libparallax.so, the gfx950 (MI355X) forward pass of
 * Parallax attention, and the causal-prefill backward pass.
 *
 * The operation.  For every query row i the library returns
 *
 *     o_i = o^SA_i - Sigma^(i)_KV rho_i
 *
 * where o^SA_i is standard softmax attention of q_i over its keys/values,
 * Sigma^(i)_KV is the KV covariance under query i's softmax weights, and
 * rho_i is the learned probe of the row (gist.science technical summary of
 * Parallax, "Method: Parallax / core mechanism", output equation).  The
 * boundary-amplification factor is fixed at zero (same page, "key design
 * choices"; news.chathome.org article, "How does the mechanism work?"), so no
 * other term is added.  A zero probe gives softmax attention exactly (the
 * news.chathome.org article, "How does the mechanism work?").
 *
 * Conventions that the pages leave open (readings):
 *   - Sigma^(i)_KV[a][b] = sum_j p_ij (v_j[a] - mean_v[a]) (k_j[b] - mean_k[b]):
 *     population form, rows index the value coordinate, columns the key
 *     coordinate, so rho has the head dimension d of the keys.
 *   - The softmax scale multiplies q.k only; rho.k is not scaled.
 *   - GQA: query head h reads KV head h / (Hq / Hkv).  rho has one probe per
 *     query head.
 *   - Prefill is causal: token t attends keys 0..t, the diagonal included.
 *   - Decode: the query attends every cached key of its sequence (its own
 *     key/value already appended).  An empty sequence returns zeros.
 *
 * Computation.  Both entry points stream K/V once (news.chathome.org article,
 * "Hardware argument"; gist.science summary, "Hardware-aware algorithm"):
 * the softmax branch and the probe branch share the K/V tiles, the running
 * max and the rescale factors.  The kernels accumulate
 *     l = sum_j P_j,  A = sum_j P_j v_j,  B = sum_j P_j r_j v_j,  c = sum_j P_j r_j
 * with P_j = exp(s_j - m), r_j = <rho, k_j>, and finish with
 *     o = A/l - (B/l - (c/l) A/l)
 * which equals the covariance form.  Accumulation is fp32.
 *
 * Memory.  Every pointer argument named as "device" is device memory owned by
 * the caller; the library never allocates, frees or synchronises.  Calls are
 * asynchronous on `stream` (NULL is the null stream) and
 * return as soon as the kernels are queued.  A device fault surfaces at the
 * caller's next synchronisation.  All tensors are dense, row-major, with the
 * head dimension innermost, and start on a 16-byte boundary (cu_seqlens: 8
 * bytes).  `out` must not overlap any input.  The library
 * is stateless and re-entrant; concurrent calls are safe if their `out` and
 * `workspace` buffers differ.
 *
 * Errors.  Arguments are checked on the host before any HIP call; a rejected
 * call returns its code and touches nothing.  After the launches,
 * hipGetLastError() != hipSuccess returns PLX_ERR_HIP.  No C++ exception
 * crosses this interface.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PLX_OK = 0,
    PLX_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad size, bad scale */
    PLX_ERR_UNSUPPORTED = 2,         /* valid but not built: head dim, group size, dtype */
    PLX_ERR_WORKSPACE_TOO_SMALL = 3, /* decode workspace below the size query */
    PLX_ERR_HIP = 4,                 /* a launch failed (hipGetLastError) */
    /* Not a status: widens the type's range to every 32-bit value, so that
     * any int a caller passes (say to parallax_status_string) is a valid
     * value of the type in C++ as in C. */
    PLX_STATUS_RANGE_ = 0x7fffffff
} plx_status_t;

typedef enum {
    PLX_DTYPE_F32 = 0,   /* IEEE float32 inputs and output */
    PLX_DTYPE_BF16 = 1,  /* bfloat16 inputs and output (round to nearest even) */
    PLX_DTYPE_RANGE_ = 0x7fffffff  /* not a dtype: as PLX_STATUS_RANGE_ */
} plx_dtype_t;

/*
 * Causal prefill (T query tokens over the same T keys): the forward pass of
 * the layer over a whole sequence, as in language-model pretraining (the
 * news.chathome.org article, "Experiments"), with the probe rho = W_R x given
 * as an input (same article, "What is Parallax"; gist.science summary,
 * "Method: Parallax / core mechanism").
 *
 *   q, rho, out : device, [B, Hq, T, d]
 *   k, v        : device, [B, Hkv, T, d]
 *   rho         : may be NULL, which selects the softmax-only kernel; its
 *                 output is bitwise equal to that of a rho of all zeros.
 *   softmax_scale: tau > 0 and finite (usually 1/sqrt(d)).
 *   dtype       : PLX_DTYPE_BF16 or PLX_DTYPE_F32, shared by all tensors.
 *
 * Supported: d in {64, 128}; Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8};
 * B, T >= 1.  Offsets are 64-bit, so tensors may exceed 2^31 elements.
 * Returns PLX_ERR_INVALID_ARGUMENT for null q/k/v/out, non-positive sizes,
 * Hq not a multiple of Hkv or a bad scale; PLX_ERR_UNSUPPORTED for other d,
 * group sizes or dtypes.
 */
plx_status_t parallax_fwd_prefill(const void *q, const void *k, const void *v,
                                  const void *rho, void *out,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                  int32_t d, float softmax_scale,
                                  plx_dtype_t dtype, hipStream_t stream);

/*
 * Causal prefill forward that also keeps what parallax_bwd_prefill needs
 * (the training forward; the pages pretrain with this layer, news.chathome.org
 * article, "Experiments").  Same inputs, output and conventions as
 * parallax_fwd_prefill, bf16 only, plus:
 *
 *   out_sa : device, [B, Hq, T, d] bf16: the softmax-attention part o^SA =
 *            A/l of each row.  Required with rho, must be NULL without it
 *            (then o^SA is out itself).
 *   lse    : device, [B, Hq, T] fp32: log2 of sum_j 2^(s_ij log2 e), with
 *            s_ij = softmax_scale * q_i.k_j over the row's causal keys, so that
 *            p_ij = 2^(s_ij log2 e - lse_i).
 *   rbar   : device, [B, Hq, T] fp32: rbar_i = sum_j p_ij (rho_i . k_j).
 *            Required with rho, must be NULL without it (then rbar = 0).
 *
 * Returns PLX_ERR_INVALID_ARGUMENT for a null lse, out_sa or rbar given
 * without rho (or missing with it), or any output overlapping an input or
 * another output; PLX_ERR_UNSUPPORTED for dtype != PLX_DTYPE_BF16; otherwise
 * as parallax_fwd_prefill.
 */
plx_status_t parallax_fwd_prefill_train(const void *q, const void *k,
                                        const void *v, const void *rho,
                                        void *out, void *out_sa, float *lse,
                                        float *rbar, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t T, int32_t d,
                                        float softmax_scale, plx_dtype_t dtype,
                                        hipStream_t stream);

/*
 * Bytes of device workspace parallax_bwd_prefill needs: 16 bytes per query
 * row, B * Hq * T * 16.  Returns SIZE_MAX for non-positive sizes.
 */
size_t parallax_bwd_prefill_workspace_size(int32_t B, int32_t Hq, int32_t T);

/*
 * Causal prefill backward: the gradients of sum(dout * o) with respect to
 * q, k, v and rho, for the forward above.  The pages print no backward pass;
 * writing the forward as o_i = sum_j w_ij v_j with
 * w_ij = p_ij (1 - r_ij + rbar_i) and r_ij = rho_i . k_j, differentiation
 * gives, with g_ij = dout_i . v_j, G_i = dout_i . o^SA_i and
 * D_i = dout_i . o_i + rbar_i G_i:
 *
 *     dS_ij = p_ij (g_ij (1 - r_ij + rbar_i) + G_i r_ij - D_i)
 *     dR_ij = p_ij (G_i - g_ij)
 *     dq_i = tau sum_j dS_ij k_j          drho_i = sum_j dR_ij k_j
 *     dk_j = tau sum_i dS_ij q_i + sum_i dR_ij rho_i
 *     dv_j = sum_i w_ij dout_i
 *
 * (dk and dv of a KV head sum over its Hq / Hkv query heads).
 *
 *   q, k, v, rho : the forward's inputs (rho NULL: softmax-only backward)
 *   out, out_sa, lse, rbar : the outputs of parallax_fwd_prefill_train
 *                  (out_sa and rbar NULL exactly when rho is)
 *   dout         : device, [B, Hq, T, d] bf16, upstream gradient
 *   dq, drho     : device, [B, Hq, T, d] bf16 outputs (drho NULL exactly
 *                  when rho is)
 *   dk, dv       : device, [B, Hkv, T, d] bf16 outputs
 *   workspace    : device, at least parallax_bwd_prefill_workspace_size
 *                  bytes, 16-byte aligned; scratch, contents not kept
 *
 * Two kernels run on `stream`: dq/drho, which also leaves each row's
 * statistics in the workspace, then dk/dv.  Every gradient is written in full (no accumulation
 * into the outputs).  Accumulation is fp32; p, w, dS and dR are rounded to
 * bf16 as matrix-core operands.
 *
 * Returns PLX_ERR_INVALID_ARGUMENT for null required pointers, a NULL pattern
 * that does not match rho's, misaligned pointers, non-positive sizes, a bad
 * scale, or an output overlapping an input, another output or the
 * workspace; PLX_ERR_WORKSPACE_TOO_SMALL; PLX_ERR_UNSUPPORTED for
 * dtype != PLX_DTYPE_BF16, other d or group sizes, or T * (Hq / Hkv) >= 2^31.
 */
plx_status_t parallax_bwd_prefill(const void *q, const void *k, const void *v,
                                  const void *rho, const void *out,
                                  const void *out_sa, const float *lse,
                                  const float *rbar, const void *dout,
                                  void *dq, void *dk, void *dv, void *drho,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                  int32_t d, float softmax_scale,
                                  plx_dtype_t dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Fused q/k/v/probe projection: the probe is a learned linear map of the
 * layer input, rho = W_R x (news.chathome.org article, "What is Parallax";
 * gist.science summary, "Method: Parallax / core mechanism"), computed as one
 * more block of output features of the q/k/v projection.  No bias.
 *
 *   x   : device, [B, T, d_model] bf16 (tokens row-major)
 *   w   : device, [(2 Hq + 2 Hkv) d, d_model] bf16, one row per output
 *         feature (a torch Linear weight): rows 0 .. Hq d - 1 are q (feature
 *         h d + a is dim a of query head h), then Hkv d rows of k, Hkv d rows
 *         of v, Hq d rows of rho.
 *   q, rho : device, [B, Hq, T, d] bf16 outputs;  k, v : [B, Hkv, T, d].
 *
 * Each output element is sum_c w[f][c] x[t][c] accumulated in fp32 and
 * rounded once to bf16 (RNE).  Supported: bf16, d in {64, 128}, d_model a
 * multiple of 64.  Returns PLX_ERR_INVALID_ARGUMENT for null or misaligned
 * pointers, non-positive sizes, or an output overlapping an input or another
 * output; PLX_ERR_UNSUPPORTED for other dtypes, d or d_model.
 */
plx_status_t parallax_qkvr_projection(const void *x, const void *w, void *q,
                                      void *k, void *v, void *rho, int32_t B,
                                      int32_t T, int32_t d_model, int32_t Hq,
                                      int32_t Hkv, int32_t d,
                                      plx_dtype_t dtype, hipStream_t stream);

/*
 * Decode: one query token per sequence over a KV cache.  Parallax keeps the
 * softmax form, so decoding reads a KV cache as softmax attention does (the
 * zubnet.ai news item on Parallax, mechanism paragraph), and each decode step
 * supplies a single query row per head (the news.chathome.org article,
 * "Hardware argument").  The library chooses how each sequence is cut into
 * chunks (one workgroup each, merged by a second kernel when there are
 * several); parallax_fwd_decode_chunked takes that choice from the caller.
 *
 *   q, rho, out : device, [B, Hq, d]; rho may be NULL (softmax only, bitwise
 *                 equal to a zero probe).
 *   k_cache, v_cache : device; may be NULL when max_ctx == 0 (every
 *                 sequence is empty and no key is read).
 *       cu_seqlens == NULL: contiguous cache [B, Hkv, max_ctx, d]; every
 *                 sequence has max_ctx keys.
 *       cu_seqlens != NULL: device int64 [B + 1] token offsets, cu[0] = 0,
 *                 non-decreasing; sequence b has L_b = cu[b+1] - cu[b] keys,
 *                 stored as a slab [Hkv, L_b, d] that starts at element
 *                 cu[b] * Hkv * d of k_cache / v_cache.  The caller promises
 *                 L_b <= max_ctx (keys past max_ctx are not read) and a
 *                 well-formed cu_seqlens (it lives on the device and is not
 *                 checked).
 *   max_ctx     : >= 0; the longest context.
 *   softmax_scale: tau > 0 and finite (usually 1/sqrt(d)).
 *   workspace   : device, at least parallax_fwd_decode_workspace_size(...)
 *                 bytes (may be NULL when that size is 0); holds the
 *                 per-chunk partial results; contents are scratch.
 *
 * Supported: d in {64, 128}; Hq / Hkv in {1, 2, 4, 8}; dtype BF16 (F32 is
 * accepted as a debugging aid).  Returns PLX_ERR_INVALID_ARGUMENT for null
 * q/out (or null k/v with max_ctx > 0), misaligned pointers, non-positive
 * sizes, Hq not a multiple of Hkv, a bad scale or an output overlapping an
 * input or the workspace; PLX_ERR_UNSUPPORTED for other d, group sizes or
 * dtypes, or more than 2^31 - 1 workgroups; PLX_ERR_WORKSPACE_TOO_SMALL.
 */
plx_status_t parallax_fwd_decode(const void *q, const void *rho,
                                 const void *k_cache, const void *v_cache,
                                 const int64_t *cu_seqlens, int64_t max_ctx,
                                 void *out, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t d, float softmax_scale,
                                 plx_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace parallax_fwd_decode needs for these sizes: 0 when
 * the library runs one chunk per sequence (no merge), and (size_t)-1 for
 * arguments parallax_fwd_decode would reject.
 */
size_t parallax_fwd_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t d, int64_t max_ctx,
                                          plx_dtype_t dtype);

/* Keys per chunk that parallax_fwd_decode uses for these sizes, or a
 * negative plx_status_t value for rejected arguments. */
int32_t parallax_fwd_decode_auto_split(int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t d, int64_t max_ctx);

/*
 * parallax_fwd_decode with the chunking chosen by the caller: each sequence
 * is cut into chunks of keys_per_split keys, one workgroup each, and the
 * chunks are merged by a second kernel (the associative merge of the
 * per-chunk softmax states).  Any setting gives the same result up to fp32
 * rounding.  For tests, sweeps and tuning; parallax_fwd_decode picks the
 * setting itself.
 *
 *   keys_per_split: 0 = the library's choice (then the call is exactly
 *                 parallax_fwd_decode); otherwise a multiple of 32 in
 *                 [32, 2^20].
 *   workspace   : at least parallax_fwd_decode_chunked_workspace_size(...,
 *                 keys_per_split) bytes.
 *
 * Other arguments, errors and conventions as parallax_fwd_decode; a
 * keys_per_split outside the range returns PLX_ERR_INVALID_ARGUMENT.
 */
plx_status_t parallax_fwd_decode_chunked(const void *q, const void *rho,
                                         const void *k_cache,
                                         const void *v_cache,
                                         const int64_t *cu_seqlens,
                                         int64_t max_ctx, void *out, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d,
                                         float softmax_scale, plx_dtype_t dtype,
                                         int32_t keys_per_split,
                                         void *workspace,
                                         size_t workspace_bytes,
                                         hipStream_t stream);

/* Workspace bytes of parallax_fwd_decode_chunked for this keys_per_split
 * (0 = the library's choice), or (size_t)-1 for rejected arguments. */
size_t parallax_fwd_decode_chunked_workspace_size(int32_t B, int32_t Hq,
                                                  int32_t Hkv, int32_t d,
                                                  int64_t max_ctx,
                                                  plx_dtype_t dtype,
                                                  int32_t keys_per_split);

/*
 * Decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, chunking, result (bit for bit) and
 * errors as parallax_fwd_decode, minus the workspace: the per-chunk partials
 * go to a scratch buffer of PLX_DECODE_NOALLOC_SCRATCH_BYTES that the library
 * holds on each device it runs on, from the first call there until the
 * process ends.  The first call on a device resolves that buffer's address
 * (hipGetSymbolAddress); no call allocates or frees anything.
 *
 * Every call on one device shares its buffer, so calls that overlap in time
 * on one device race (two streams, or two host threads): serialise them.  A
 * call whose workspace size (parallax_fwd_decode_workspace_size) exceeds the
 * buffer returns PLX_ERR_WORKSPACE_TOO_SMALL before any HIP call; every
 * contiguous or ragged cache of up to 2^20 keys fits.
 */
#define PLX_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

plx_status_t parallax_fwd_decode_noalloc(const void *q, const void *rho,
                                         const void *k_cache,
                                         const void *v_cache,
                                         const int64_t *cu_seqlens,
                                         int64_t max_ctx, void *out, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d,
                                         float softmax_scale, plx_dtype_t dtype,
                                         hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *parallax_status_string(plx_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
