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

// Two floats -> packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

}  // namespace lisa
