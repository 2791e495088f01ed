// Device helpers shared by the LISA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

typedef uint16_t bf16_t;  // bfloat16 storage bits

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 16-byte vector of elements of T converted to fp32.
template <typename T> struct Vec;

template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static void load(const float* p, float (&f)[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&f)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ __forceinline__ static void load(const bf16_t* p, float (&f)[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float (&f)[8]) {
    uint4 v;
    v.x = f2bf(f[0]) | (f2bf(f[1]) << 16);
    v.y = f2bf(f[2]) | (f2bf(f[3]) << 16);
    v.z = f2bf(f[4]) | (f2bf(f[5]) << 16);
    v.w = f2bf(f[6]) | (f2bf(f[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void st1(T* p, float v);
template <> __device__ __forceinline__ void st1<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st1<bf16_t>(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }

// Raw 16-byte load (unpacked later with Vec<T>::unpack).
template <typename T> __device__ __forceinline__ uint4 ld16(const T* p) { return *reinterpret_cast<const uint4*>(p); }

// elu(x) + 1
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

__device__ __forceinline__ float sigmoidf(float a) { return 1.f / (1.f + __expf(-a)); }

// Partner value of a butterfly level inside a wave.  Levels 1 and 2 swap
// lanes inside a quad (DPP quad_perm); levels 4 and 8 mirror 8- and 16-lane
// rows (DPP row_half_mirror / row_mirror), which equals the xor partner's
// value once the lower levels have made each aligned group uniform; levels
// 16 and 32 go through the LDS crossbar.
template <int LEVEL>
__device__ __forceinline__ float butterfly_partner(float v) {
  const int x = __float_as_int(v);
  if constexpr (LEVEL == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  else if constexpr (LEVEL == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  else if constexpr (LEVEL == 4) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true));
  else if constexpr (LEVEL == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true));
  else return __shfl_xor(v, LEVEL, WAVE);
}

// Sum over aligned groups of `hi` lanes of values that are already uniform
// inside aligned groups of `lo` lanes (lo, hi powers of two, lo <= hi <= 64;
// lo = 1 for a plain group sum).  Every lane of a group receives the sum.
// The uniformity precondition matters: levels 4 and 8 pair lane i with its
// mirror, not with lane i ^ 4 or i ^ 8.
// The width tests are wave-uniform, so they cost scalar branches only.
__device__ __forceinline__ float group_sum_range(float v, int lo, int hi) {
  if (lo <= 1 && hi > 1) v += butterfly_partner<1>(v);
  if (lo <= 2 && hi > 2) v += butterfly_partner<2>(v);
  if (lo <= 4 && hi > 4) v += butterfly_partner<4>(v);
  if (lo <= 8 && hi > 8) v += butterfly_partner<8>(v);
  if (lo <= 16 && hi > 16) v += butterfly_partner<16>(v);
  if (lo <= 32 && hi > 32) v += butterfly_partner<32>(v);
  return v;
}
__device__ __forceinline__ float group_sum(float v, int width) { return group_sum_range(v, 1, width); }

// Sum over the lanes that share (lane mod 8): true xor partners 8, 16, 32
// (DPP row_ror:8 swaps the two halves of a 16-lane row).
__device__ __forceinline__ float sum_lanes_mod8(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
  v += __shfl_xor(v, 16, WAVE);
  v += __shfl_xor(v, 32, WAVE);
  return v;
}

__device__ __forceinline__ float group_max(float v, int width) {
  if (width > 1) v = fmaxf(v, butterfly_partner<1>(v));
  if (width > 2) v = fmaxf(v, butterfly_partner<2>(v));
  if (width > 4) v = fmaxf(v, butterfly_partner<4>(v));
  if (width > 8) v = fmaxf(v, butterfly_partner<8>(v));
  if (width > 16) v = fmaxf(v, butterfly_partner<16>(v));
  if (width > 32) v = fmaxf(v, butterfly_partner<32>(v));
  return v;
}

// ---------------------------------------------------------------------------
// Wave-wide primitives on DPP row operations (a wave is four 16-lane rows);
// the four row results are combined through readlane, so the result is a
// wave-uniform value.  No LDS crossbar round trips.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
// row_shr:N with zero fill for lanes whose source lies before the row
template <int N>
__device__ __forceinline__ uint32_t dpp_shr_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t rl(uint32_t v, int lane) { return (uint32_t)__builtin_amdgcn_readlane((int)v, lane); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  return max(max(rl(v, 0), rl(v, 16)), max(rl(v, 32), rl(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  return min(min(rl(v, 0), rl(v, 16)), min(rl(v, 32), rl(v, 48)));
}
// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_shr_u32<1>(v);
  v += dpp_shr_u32<2>(v);
  v += dpp_shr_u32<4>(v);
  v += dpp_shr_u32<8>(v);
  const uint32_t r0 = rl(v, 15), r1 = rl(v, 31), r2 = rl(v, 47);
  const int row = (threadIdx.x & (WAVE - 1)) >> 4;
  v += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return v;
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key).
// -0.0 is folded onto +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Log-sum-exp pairs: (m, s) stands for a set of logits with max m and
// sum of exp(logit - m) s (m = -inf, s = 0 for the empty set).  Merging two
// pairs gives the pair of the union.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void lse_merge_xor(float& m, float& s, int mask) {
  const float m2 = __shfl_xor(m, mask, WAVE), s2 = __shfl_xor(s, mask, WAVE);
  lse_merge(m, s, m2, s2);
}

// Block-wide sum / max of one value per thread (256 threads); every thread
// receives the result.  `red` holds four floats and is free again on return.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = group_sum(v, WAVE);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_max256(float v, float* red) {
  v = group_max(v, WAVE);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = v;
  __syncthreads();
  const float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return s;
}

}  // namespace lisa
