// bf16 MFMA helpers for gfx950 (wave64).
//
// v_mfma_f32_16x16x32_bf16 operand layout (lane l, v = 0..7, r = 0..3):
//   A (16 x 32, rows i):    lane l holds A[l % 16][8 * (l / 16) + v]
//   B (32 x 16, cols j):    lane l holds B[8 * (l / 16) + v][l % 16]
//   C/D (16 x 16):          lane l holds D[4 * (l / 16) + r][l % 16]
// So an A fragment is 8 consecutive elements of one row of a row-major
// [rows][K] array, and a B fragment 8 consecutive elements of one row of the
// transposed [cols][K] array: both are single 16-byte reads.
#pragma once
#include "lisa_common.h"

namespace lisa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 lds_read16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even; one instruction on
// gfx950), low half first.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// a = hi + lo and b likewise to about 2^-17: hi = bf16(x), lo = bf16(x - hi),
// as packed pairs (a in the low halves).
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

}  // namespace lisa
