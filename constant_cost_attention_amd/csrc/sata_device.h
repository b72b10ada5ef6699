// Device-side helpers for the gfx950 SATA kernels: dtype conversion, MFMA
// wrappers and the monomial expansion shared by every kernel.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sata {

typedef uint16_t bf16_t;                                     // bfloat16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));   // MFMA operand, 8 x bf16
typedef float f32x4 __attribute__((ext_vector_type(4)));     // MFMA accumulator, 16x16 tile

typedef _Float16 f16_t;                                      // IEEE binary16 storage

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    __bf16 b = (__bf16)x;                                    // round to nearest even
    return __builtin_bit_cast(bf16_t, b);
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }   // nearest even

// Packed feature tuple (see sata_internal.h): four index slots, unused ones
// pointing at the constant-1 slot.
__device__ __forceinline__ int tup_i1(uint32_t t) { return (int)(t & 0xffu); }
__device__ __forceinline__ int tup_i2(uint32_t t) { return (int)((t >> 8) & 0xffu); }
__device__ __forceinline__ int tup_i3(uint32_t t) { return (int)((t >> 16) & 0xffu); }
__device__ __forceinline__ int tup_i4(uint32_t t) { return (int)(t >> 24); }

// Monomial prod_r x[i_r] of one feature, reading x from an array laid out with
// `stride` between consecutive dims; slot d_K holds 1 and slot d_K+1 holds 0
// [hotdry, "Engineering realisation of the constant compute cost": keys (and
// queries) are mapped to the minimal-basis features through M_p].
__device__ __forceinline__ float monomial(uint32_t t, const float *x, int stride) {
    return x[tup_i1(t) * stride] * x[tup_i2(t) * stride] * x[tup_i3(t) * stride] * x[tup_i4(t) * stride];
}
// The same with the first NF slots only, for index tables of features of
// degree below NF + 1 (P <= NF: the remaining slots hold the constant 1).
template <int NF> __device__ __forceinline__ float monomial_n(uint32_t t, const float *x, int stride) {
    static_assert(NF == 3 || NF == 4, "three or four slots");
    const float m = x[tup_i1(t) * stride] * x[tup_i2(t) * stride] * x[tup_i3(t) * stride];
    if constexpr (NF == 4) return m * x[tup_i4(t) * stride];
    return m;
}

// ---- MFMA -------------------------------------------------------------------
// 16x16x32 bf16 (gfx950): lane l holds A[l%16][8*(l/16) + 0..7],
// B[8*(l/16) + 0..7][l%16]; accumulator lane l holds D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: lane l holds A[l%16][l/16], B[l/16][l%16]; same accumulator.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// two floats -> bf16 pair (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Lane 4 * (lane / 4) + X's value of x, for every lane (DPP quad broadcast; folds into the
// consuming VALU operation's source).
template <int X>
__device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), X * 0x55, 0xf, 0xf, true));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
    return r;
}

}  // namespace sata
