// bf16 MFMA prefill kernels for the indexer scores and the gate logits.
//
//  * index scores ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2):
//    s[t, j] = sum_h w_h ReLU(q_I[t,h] . k_I[j, h H_Ik / H_I]) for the
//    stored rows t and every key j <= t.  Per head the dot products are one
//    MFMA contraction over d_I; ReLU and w_h are applied to the fp32 result.
//    Tiles are computed transposed (keys along the accumulator rows) so that
//    each lane holds four consecutive keys of one query row and stores them
//    as one float4.  Query and key rows are staged in LDS per head.
//  * gate logits (Section 3.3 Eq. 5): x[row] . W_g[:, h] as one GEMM over
//    the hidden dimension; the sigmoid is applied where the gate is used.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"
#include "lisa_prefill.h"

namespace lisa {

// ---------------------------------------------------------------------------
// index scores: block = 128 query rows x 128 keys, wave = 64 x 64 (4 x 4
// tiles of 16 x 16).  Per indexer head the block stages the head's query and
// key rows in LDS (the next head's rows are loaded into registers meanwhile),
// and every wave reads its MFMA operands from there.
// ---------------------------------------------------------------------------
constexpr int IX_T = 128;          // query rows and keys per block
constexpr int IX_PAD = 8;

template <int DI>
struct IndexShared {
  bf16_t q[IX_T][DI + IX_PAD];
  bf16_t k[IX_T][DI + IX_PAD];
};

template <int DI>
__global__ __launch_bounds__(256) void k_index_scores_mfma(IndexScoreArgs a) {
  __shared__ IndexShared<DI> sm;
  const Shape& sh = a.sh;
  const int b = blockIdx.z;
  const int T0 = IX_T * blockIdx.y, J0 = IX_T * blockIdx.x;
  if (J0 > T0 + IX_T - 1 || T0 + IX_T <= a.row0) return;  // above the diagonal / not stored
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int tw = T0 + 64 * (wave >> 1), jw = J0 + 64 * (wave & 1);
  const bool live = jw <= tw + 63;  // some key of the wave's tiles is causal for some row
  const int R = sh.H_I / sh.H_Ik;
  const bf16_t* qb = (const bf16_t*)a.q_idx + (size_t)b * a.n * sh.H_I * DI;
  const bf16_t* kb = (const bf16_t*)a.k_idx + (size_t)b * sh.cap * sh.H_Ik * DI;

  // staging: the block's 128 rows of one head, DI / 8 vectors of 16 B each
  constexpr int NV = IX_T * DI / 8 / 256;
  uint4 rq[NV], rk[NV];
  auto fetch = [&](int h) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = tid + 256 * m;
      const int row = e / (DI / 8), c8 = e % (DI / 8);
      rq[m] = ld16(qb + ((size_t)min(T0 + row, a.n - 1) * sh.H_I + h) * DI + 8 * c8);
      rk[m] = ld16(kb + ((size_t)min(J0 + row, a.n - 1) * sh.H_Ik + h / R) * DI + 8 * c8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = tid + 256 * m;
      const int row = e / (DI / 8), c8 = e % (DI / 8);
      *reinterpret_cast<uint4*>(&sm.q[row][8 * c8]) = rq[m];
      *reinterpret_cast<uint4*>(&sm.k[row][8 * c8]) = rk[m];
    }
  };

  f32x4 sc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[i][c] = zero4();
  const int qr0 = 64 * (wave >> 1), kr0 = 64 * (wave & 1);  // the wave's rows in the staged tiles
  fetch(0);
  for (int h = 0; h < sh.H_I; ++h) {
    __syncthreads();  // readers of the previous head are done
    stage();
    __syncthreads();
    if (h + 1 < sh.H_I) fetch(h + 1);
    if (!live) continue;
    const float w = a.w_idx[h];
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DI; k0 += 32) {
      bf16x8 qf[4], kf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = as_bf16x8(lds_read16(&sm.q[qr0 + 16 * i + r16][k0 + 8 * g]));
#pragma unroll
      for (int c = 0; c < 4; ++c) kf[c] = as_bf16x8(lds_read16(&sm.k[kr0 + 16 * c + r16][k0 + 8 * g]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = mfma16(kf[c], qf[i], acc[i][c]);  // [key][query]
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[i][c][r] = fmaf(w, fmaxf(acc[i][c][r], 0.f), sc[i][c][r]);
  }
  if (!live) return;
  // lane holds s[t = tw + 16 i + r16][j = jw + 16 c + 4 g + r]; keys past t are written as 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tw + 16 * i + r16;
    if (t < a.row0 || t >= a.n) continue;
    float* orow = a.scores + ((size_t)b * a.stored_rows + (t - a.row0)) * a.ld;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = jw + 16 * c + 4 * g;
      if (j > t) continue;
      float4 v;
      v.x = sc[i][c][0];
      v.y = j + 1 <= t ? sc[i][c][1] : 0.f;
      v.z = j + 2 <= t ? sc[i][c][2] : 0.f;
      v.w = j + 3 <= t ? sc[i][c][3] : 0.f;
      *reinterpret_cast<float4*>(orow + j) = v;
    }
  }
}

bool index_mfma_supported(const Shape& sh) { return sh.dtype == 1 && (sh.d_I == 32 || sh.d_I == 64 || sh.d_I == 128); }

hipError_t launch_index_scores_mfma(const IndexScoreArgs& a, hipStream_t st) {
  if (a.n - a.row0 <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n + IX_T - 1) / IX_T), (unsigned)((a.n + IX_T - 1) / IX_T), (unsigned)a.sh.B);
  switch (a.sh.d_I) {
    case 32: klaunch(k_index_scores_mfma<32>, grid, dim3(256), 0, st, a); break;
    case 64: klaunch(k_index_scores_mfma<64>, grid, dim3(256), 0, st, a); break;
    default: klaunch(k_index_scores_mfma<128>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gate logits: W_g [hidden, H_q] is first transposed into [H_pad, hidden]
// (H_pad = H_q rounded up to 16, zero rows) so that both MFMA operands are
// 16-byte row reads; block = 64 rows, wave = 16 rows x H_pad heads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gate_transpose(GateArgs a) {
  const Shape& sh = a.sh;
  const int hp = (sh.H_q + 15) / 16 * 16;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)hp * sh.hidden) return;
  const int h = (int)(e / sh.hidden), c = (int)(e % sh.hidden);
  a.w_t[e] = h < sh.H_q ? ((const bf16_t*)a.w_gate)[(size_t)c * sh.H_q + h] : (bf16_t)0;
}

template <int NH>  // head tiles of 16
__global__ __launch_bounds__(256) void k_gate_mfma(GateArgs a) {
  const Shape& sh = a.sh;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 64 + 16 * wave;
  if (row0 >= a.n_rows) return;
  const int row = min(row0 + r16, a.n_rows - 1);
  const bf16_t* x = (const bf16_t*)a.x + (size_t)row * sh.hidden + 8 * g;
  const bf16_t* w = a.w_t + (size_t)r16 * sh.hidden + 8 * g;
  f32x4 acc[NH];
#pragma unroll
  for (int q = 0; q < NH; ++q) acc[q] = zero4();
  int c = 0;
  for (; c + 64 <= sh.hidden; c += 64) {  // two K steps per iteration, loads first
    uint4 xv[2], wv[2][NH];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      xv[s] = ld16(x + c + 32 * s);
#pragma unroll
      for (int q = 0; q < NH; ++q) wv[s][q] = ld16(w + (size_t)16 * q * sh.hidden + c + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int q = 0; q < NH; ++q) acc[q] = mfma16(as_bf16x8(wv[s][q]), as_bf16x8(xv[s]), acc[q]);
  }
  for (; c < sh.hidden; c += 32) {
    const uint4 xv = ld16(x + c);
#pragma unroll
    for (int q = 0; q < NH; ++q)
      acc[q] = mfma16(as_bf16x8(ld16(w + (size_t)16 * q * sh.hidden + c)), as_bf16x8(xv), acc[q]);
  }
  // lane holds logit[row0 + r16][h = 16 q + 4 g + r]
  if (row0 + r16 < a.n_rows) {
    float* o = a.gate_part + (size_t)(row0 + r16) * sh.H_q;
#pragma unroll
    for (int q = 0; q < NH; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * q + 4 * g + r;
        if (h < sh.H_q) o[h] = acc[q][r];
      }
  }
}

bool gate_mfma_supported(const Shape& sh) { return sh.dtype == 1 && sh.hidden % 32 == 0 && sh.H_q <= 64; }

size_t gate_transpose_elems(const Shape& sh) { return (size_t)((sh.H_q + 15) / 16 * 16) * sh.hidden; }

hipError_t launch_gate_transpose(const GateArgs& a, hipStream_t st) {
  const size_t te = gate_transpose_elems(a.sh);
  klaunch(k_gate_transpose, dim3((unsigned)((te + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gate_mfma(const GateArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_rows + 63) / 64));
  switch ((a.sh.H_q + 15) / 16) {
    case 1: klaunch(k_gate_mfma<1>, grid, dim3(256), 0, st, a); break;
    case 2: klaunch(k_gate_mfma<2>, grid, dim3(256), 0, st, a); break;
    case 3: klaunch(k_gate_mfma<3>, grid, dim3(256), 0, st, a); break;
    default: klaunch(k_gate_mfma<4>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace lisa
