// plx_device.h -- gfx950 device building blocks shared by the Parallax decode
// and prefill kernels: element types, 8-element MFMA operands, the k = 32
// matrix-core step, operand packing and wavefront reductions.
//
// Matrix-core layout used throughout (v_mfma_f32_16x16x32_bf16 and the fp32
// v_mfma_f32_16x16x4_f32 issued eight times over the same 32-wide slice):
//   lane l, col = l % 16, grp = l / 16
//   A operand (16 x 32): lane holds row `col`, contraction slots 8*grp .. 8*grp+7
//   B operand (32 x 16): lane holds column `col`, the same 8 contraction slots
//   C/D (16 x 16, fp32): lane holds rows 4*grp .. 4*grp+3 of column `col`
// Which data index each contraction slot stands for is free as long as A and
// B agree; the kernels use that freedom so that every lane's 8 operand
// elements are contiguous in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));

constexpr int kWave = 64;

// Element type tags.  Storage is the raw element as it sits in memory.
struct BF16 {
    using storage = uint16_t;
};
struct F32 {
    using storage = float;
};

// Eight consecutive contraction elements of one lane.
template <class T> struct Op8;
template <> struct Op8<BF16> {
    u32x4 w;  // element e in half (e & 1) of word e >> 1
};
template <> struct Op8<F32> {
    float v[8];
};

__device__ __forceinline__ Op8<BF16> op8_zero(BF16) {
    Op8<BF16> o;
    o.w = u32x4{0u, 0u, 0u, 0u};
    return o;
}
__device__ __forceinline__ Op8<F32> op8_zero(F32) {
    Op8<F32> o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = 0.f;
    return o;
}

// Eight consecutive elements from global or shared memory (16-byte aligned
// for bf16, 32-byte aligned for fp32).
__device__ __forceinline__ Op8<BF16> op8_load(const uint16_t *p) {
    Op8<BF16> o;
    o.w = *reinterpret_cast<const u32x4 *>(p);
    return o;
}
// Streaming form for data read exactly once (the decode K/V stream): a
// non-temporal load, which measured 5-12% more decode bandwidth than a
// cached one; K/V tiles that other workgroups re-read through L2 (prefill)
// keep op8_load.
__device__ __forceinline__ Op8<BF16> op8_load_stream(const uint16_t *p) {
    Op8<BF16> o;
    o.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return o;
}
__device__ __forceinline__ Op8<F32> op8_load_stream(const float *p);
__device__ __forceinline__ Op8<F32> op8_load(const float *p) {
    Op8<F32> o;
    const f32x4 a = reinterpret_cast<const f32x4 *>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4 *>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o.v[e] = a[e];
        o.v[4 + e] = b[e];
    }
    return o;
}

// Value operand from two transposing LDS reads (ds_read_b64_tr_b16).  Within
// each 16-lane group, lane j receives element j % 4 of the 8-byte rows that
// lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12 point at, in that order; `lo`
// supplies operand elements 0..3 and `hi` elements 4..7.
__device__ __forceinline__ Op8<BF16> op8_load_tr(const uint16_t *lo, const uint16_t *hi) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lo));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(hi));
    const u32x2 wa = __builtin_bit_cast(u32x2, a);
    const u32x2 wb = __builtin_bit_cast(u32x2, b);
    Op8<BF16> o;
    o.w = u32x4{wa.x, wa.y, wb.x, wb.y};
    return o;
}

// C += A * B over one 32-wide contraction slice.
__device__ __forceinline__ f32x4 mma32(const Op8<BF16> &a, const Op8<BF16> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                   __builtin_bit_cast(bf16x8, b.w), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(const Op8<F32> &a, const Op8<F32> &b, f32x4 c) {
    // Slot e of lane group grp is contraction index 8*grp + e; the k = 4
    // instruction contracts over grp, so issuing it for e = 0..7 covers all 32.
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
}

// fp32 -> storage element, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_storage(float x, BF16) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float to_storage(float x, F32) { return x; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// Two fp32 -> one packed bf16 pair (lo in bits 0..15) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Eight fp32 values -> a B operand (probabilities, probe-weighted probabilities).
__device__ __forceinline__ Op8<BF16> op8_pack(const float (&x)[8], BF16) {
    Op8<BF16> o;
    o.w = u32x4{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]),
                pack2_bf16(x[6], x[7])};
    return o;
}
__device__ __forceinline__ Op8<F32> op8_pack(const float (&x)[8], F32) {
    Op8<F32> o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = x[e];
    return o;
}

// acc + the sum of the 8 operand values exactly as the MFMA sees them (after
// rounding to bf16).  Row sums taken over these values make the weights that
// multiply V sum exactly to the normaliser, so rounding perturbs the weights
// but not their total.  For bf16 each pair is one v_dot2 against (1, 1).
__device__ __forceinline__ float op8_sum_acc(const Op8<BF16> &o, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    // Words are copied to scalars first: a bit_cast straight from a vector
    // element (o.w[j]) compiled to a read of element 0 for every j.
    const uint32_t w0 = o.w.x, w1 = o.w.y, w2 = o.w.z, w3 = o.w.w;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), one, acc, false);
    return acc;
}
__device__ __forceinline__ float op8_sum_acc(const Op8<F32> &o, float acc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += o.v[e];
    return acc;
}
template <class T>
__device__ __forceinline__ float op8_sum(const Op8<T> &o) { return op8_sum_acc(o, 0.f); }

__device__ __forceinline__ Op8<F32> op8_load_stream(const float *p) {
    Op8<F32> o;
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o.v[e] = a[e];
        o.v[4 + e] = b[e];
    }
    return o;
}

// Eight storage elements to memory (LDS or global; 16-byte aligned).
__device__ __forceinline__ void store_op8(uint16_t *dst, const Op8<BF16> &o) {
    *reinterpret_cast<u32x4 *>(dst) = o.w;
}
__device__ __forceinline__ void store_op8(float *dst, const Op8<F32> &o) {
    reinterpret_cast<f32x4 *>(dst)[0] = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
    reinterpret_cast<f32x4 *>(dst)[1] = f32x4{o.v[4], o.v[5], o.v[6], o.v[7]};
}

// Four fp32 results to four contiguous storage elements (RNE for bf16).
__device__ __forceinline__ void store4(uint16_t *dst, const float (&y)[4]) {
    *reinterpret_cast<u32x2 *>(dst) = u32x2{pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])};
}
__device__ __forceinline__ void store4(float *dst, const float (&y)[4]) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{y[0], y[1], y[2], y[3]};
}

// Wave-uniform "any lane": true on every lane if pred holds on one.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// 16-bit element `e` of a packed bf16 pair word, as the low or high half.
__device__ __forceinline__ uint32_t half_lo(uint32_t w, int e) { return (e & 1) ? (w >> 16) : (w & 0xffffu); }
__device__ __forceinline__ uint32_t half_hi(uint32_t w, int e) { return (e & 1) ? (w & 0xffff0000u) : (w << 16); }

// Value of lane (l - SH) within the same 16-lane row (DPP row_shr); lanes
// with no source get 0.  Call it where every lane is active: a source lane
// that is switched off also yields 0.
template <int SH>
__device__ __forceinline__ float row_shr(float x) {
    static_assert(SH >= 1 && SH <= 15, "row_shr distance");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + SH, 0xf, 0xf, false));
}

// Reductions over the four lane groups that hold the same column.
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float group_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace plx
