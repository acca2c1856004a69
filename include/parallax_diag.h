/*
 * parallax_diag.h -- measurement aids exported by libparallax.so beside the
 * attention entry points of parallax.h (whose status codes and stream type
 * they share).  None of the attention entry points calls them.
 *
 * They give the two ceilings against which the attention kernels' rates are
 * read: the device's own bf16 matrix-core peak, computed from its compute-unit
 * count and maximum engine clock, and measured rates of a plain streaming-read
 * kernel (the HBM side) and of a kernel that does nothing but bf16 MFMAs (the
 * matrix side).  The measured rates show what the chip sustains under load,
 * which sits below the datasheet figures (clock droop under matrix load,
 * DRAM efficiency).
 */
#ifndef PARALLAX_DIAG_H
#define PARALLAX_DIAG_H

#include "parallax.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Compute units and maximum engine clock of HIP device `device`, as the HIP
 * runtime reports them (the figures rocminfo prints).  The dense bf16
 * matrix-core peak of a gfx950 device is cu_count x clock x 4096 flop per
 * cycle (4 SIMDs, each finishing one 16x16x32 bf16 MFMA, 16384 flop, every
 * 16 cycles).
 *
 *   cu_count, max_clock_khz : host, one int32 each, written on success.
 *
 * Returns PLX_ERR_INVALID_ARGUMENT for null outputs, PLX_ERR_HIP if the
 * runtime query fails (for example, no such device).
 */
plx_status_t parallax_diag_device_info(int32_t device, int32_t *cu_count,
                                       int32_t *max_clock_khz);

/*
 * Plain streaming read: every byte of src is loaded once, in 16-byte vectors
 * (four in flight per thread, a grid-stride loop over two workgroups of 256
 * threads per compute unit), and folded into a register by XOR.  Nothing is
 * written except, in the rare case that the fold hits one fixed 64-bit
 * pattern, one word of sink, so the loads cannot be dropped.
 *
 *   src         : device, 16-byte aligned, `bytes` readable bytes.
 *   bytes       : > 0 and a multiple of 16.
 *   nontemporal : nonzero for non-temporal loads (the decode kernels' form),
 *                 zero for ordinary cached loads.
 *   sink        : device, 4 bytes, not overlapping src; its contents are
 *                 meaningless.
 *
 * Returns PLX_ERR_INVALID_ARGUMENT for null or misaligned pointers, a byte
 * count of 0 or not a multiple of 16, or an overlapping sink.
 */
plx_status_t parallax_diag_stream_read(const void *src, size_t bytes,
                                       int32_t nontemporal, void *sink,
                                       hipStream_t stream);

/*
 * Matrix-core throughput: n_blocks workgroups of 4 wavefronts, each wavefront
 * issuing `iterations` x 8 v_mfma_f32_16x16x32_bf16 over eight independent
 * accumulators, with no memory traffic inside the loop.  The work is
 * n_blocks x 4 x 8 x iterations x 16384 flop.  Two workgroups per compute
 * unit put two wavefronts on each SIMD, the occupancy of the prefill kernel.
 *
 *   sink : device, 4 bytes, written only in the rare case described for
 *          parallax_diag_stream_read.
 *
 * Returns PLX_ERR_INVALID_ARGUMENT for a null sink, n_blocks outside
 * [1, 2^20] or iterations outside [1, 2^24].
 */
plx_status_t parallax_diag_mfma_bf16(void *sink, int32_t n_blocks,
                                     int32_t iterations, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_DIAG_H */
