// Prefill kernels of the LISA layer for gfx950 (shape-generic versions).
//
//  * index scores: s[t, j] = sum_h w_h ReLU(q_I[t,h] . k_I[j, h*H_Ik/H_I])
//    for every causal pair j <= t of the stored rows ("LISA", arXiv
//    2607.19358v1, Section 3.2 Stage 2);
//  * gate logits: x[t] . W_g[:, h] (Section 3.3 Eq. 5); the attention
//    epilogue applies the sigmoid;
//  * linear branch: the token recurrence of Section 3.3 Eqs. 3-4 with
//    phi = elu + 1, one block per 32 columns of S, the state held in
//    registers for the whole sequence.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_prefill.h"

namespace lisa {

// ---------------------------------------------------------------------------
// index scores (fp32 VALU, 64 x 64 tiles, 4 x 4 scores per thread)
// ---------------------------------------------------------------------------
constexpr int IS_TILE = 64;

template <typename T>
__global__ __launch_bounds__(256) void k_index_scores_generic(IndexScoreArgs a) {
  __shared__ float qs[IS_TILE][IS_TILE + 1];
  __shared__ float ks[IS_TILE][IS_TILE + 1];
  const Shape& sh = a.sh;
  const int b = blockIdx.z;
  const int t0 = a.row0 + blockIdx.y * IS_TILE;
  const int j0 = blockIdx.x * IS_TILE;
  if (t0 >= a.n || j0 > t0 + IS_TILE - 1) return;  // outside the causal triangle
  const int tid = threadIdx.x;
  const int tr = (tid / 16) * 4, tc = (tid % 16) * 4;
  float sc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[i][k] = 0.f;
  const T* q = (const T*)a.q_idx + (size_t)b * a.n * sh.H_I * sh.d_I;
  const T* kk = (const T*)a.k_idx + (size_t)b * sh.cap * sh.H_Ik * sh.d_I;
  for (int h = 0; h < sh.H_I; ++h) {
    const int kh = (h * sh.H_Ik) / sh.H_I;
    float dot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) dot[i][k] = 0.f;
    for (int c0 = 0; c0 < sh.d_I; c0 += IS_TILE) {
      const int cw = min(IS_TILE, sh.d_I - c0);
      __syncthreads();
      for (int e = tid; e < IS_TILE * IS_TILE; e += 256) {
        const int rr = e / IS_TILE, cc = e % IS_TILE;
        const int t = t0 + rr, j = j0 + rr;
        qs[rr][cc] = (cc < cw && t < a.n) ? ld1<T>(q + ((size_t)t * sh.H_I + h) * sh.d_I + c0 + cc) : 0.f;
        ks[rr][cc] = (cc < cw && j < a.n) ? ld1<T>(kk + ((size_t)j * sh.H_Ik + kh) * sh.d_I + c0 + cc) : 0.f;
      }
      __syncthreads();
      for (int c = 0; c < cw; ++c) {
        float qv[4], kv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qv[i] = qs[tr + i][c];
          kv[i] = ks[tc + i][c];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) dot[i][k] = fmaf(qv[i], kv[k], dot[i][k]);
      }
    }
    const float w = a.w_idx[h];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[i][k] = fmaf(w, fmaxf(dot[i][k], 0.f), sc[i][k]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tr + i;
    if (t >= a.n) continue;
    float* orow = a.scores + ((size_t)b * a.stored_rows + (t - a.row0)) * a.ld;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = j0 + tc + k;
      if (j <= t) orow[j] = sc[i][k];
    }
  }
}

hipError_t launch_index_scores(const IndexScoreArgs& a, hipStream_t st) {
  const int rows = a.n - a.row0;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n + IS_TILE - 1) / IS_TILE), (unsigned)((rows + IS_TILE - 1) / IS_TILE),
                  (unsigned)a.sh.B);
  if (a.sh.dtype == 0)
    klaunch(k_index_scores_generic<float>, grid, dim3(256), 0, st, a);
  else
    klaunch(k_index_scores_generic<bf16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gate logits x[row] . W_g[:, h]: block = 64 rows, W_g staged through LDS in
// 128-row chunks; 4 threads per row, each covering 32 hidden entries per chunk
// ---------------------------------------------------------------------------
constexpr int GT_ROWS = 64;
constexpr int GT_CHUNK = 128;

int prefill_gate_chunks(const Shape&) { return 1; }

template <typename T>
__global__ __launch_bounds__(256) void k_gate_logits(GateArgs a) {
  __shared__ float ws[GT_CHUNK][GMAX_GATE];
  const Shape& sh = a.sh;
  const int row0 = blockIdx.x * GT_ROWS;
  const int tid = threadIdx.x;
  const int rr = tid / 4, part = tid % 4;
  const int row = row0 + rr;
  const T* w = (const T*)a.w_gate;
  const T* x = (const T*)a.x + (size_t)min(row, a.n_rows - 1) * sh.hidden;
  float acc[GMAX_GATE];
#pragma unroll
  for (int h = 0; h < GMAX_GATE; ++h) acc[h] = 0.f;
  for (int c0 = 0; c0 < sh.hidden; c0 += GT_CHUNK) {
    const int cw = min(GT_CHUNK, sh.hidden - c0);
    __syncthreads();
    for (int e = tid; e < GT_CHUNK * GMAX_GATE; e += 256) {
      const int c = e / GMAX_GATE, h = e % GMAX_GATE;
      ws[c][h] = (c < cw && h < sh.H_q) ? ld1<T>(w + (size_t)(c0 + c) * sh.H_q + h) : 0.f;
    }
    __syncthreads();
    const int cb = part * (GT_CHUNK / 4);
    for (int c = cb; c < cb + GT_CHUNK / 4 && c < cw; ++c) {
      const float xv = ld1<T>(x + c0 + c);
#pragma unroll
      for (int h = 0; h < GMAX_GATE; ++h) acc[h] = fmaf(xv, ws[c][h], acc[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < GMAX_GATE; ++h) {
    acc[h] += __shfl_xor(acc[h], 1, WAVE);
    acc[h] += __shfl_xor(acc[h], 2, WAVE);
  }
  if (part == 0 && row < a.n_rows) {
    float* o = a.gate_part + (size_t)row * sh.H_q;
#pragma unroll
    for (int h = 0; h < GMAX_GATE; ++h)
      if (h < sh.H_q) o[h] = acc[h];
  }
}

hipError_t launch_gate_logits(const GateArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_rows + GT_ROWS - 1) / GT_ROWS));
  if (a.sh.dtype == 0)
    klaunch(k_gate_logits<float>, grid, dim3(256), 0, st, a);
  else
    klaunch(k_gate_logits<bf16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// linear branch, token recurrence: block = (b, h, 32 columns of S)
// thread (rg = tid % 8, col = tid / 8) holds rows rg, rg+8, ... of one column
// ---------------------------------------------------------------------------
constexpr int LR_COLS = 32;
constexpr int LR_STAGE = 16;  // tokens staged in LDS at a time
constexpr int LR_DMAX = 128;

template <typename T>
__global__ __launch_bounds__(256) void k_linear_recurrent(LinearArgs a) {
  __shared__ float fks[LR_STAGE][LR_DMAX];
  __shared__ float fqs[LR_STAGE][LR_DMAX];
  __shared__ float vs[LR_STAGE][LR_COLS];
  const Shape& sh = a.sh;
  const int d = sh.d;
  const int slices = d / LR_COLS;
  int blk = blockIdx.x;
  const int slice = blk % slices;
  blk /= slices;
  const int h = blk % sh.H_L, b = blk / sh.H_L;
  const int c0 = slice * LR_COLS;
  const int tid = threadIdx.x;
  const int rg = tid % 8, col = tid / 8;
  constexpr int RMAX = LR_DMAX / 8;
  const int nr = d / 8;
  const bool normalized = !(sh.flags & 1u);

  float S[RMAX], z[RMAX];
  const size_t hs = ((size_t)b * sh.H_L + h);
  const float* S0 = a.S + hs * d * d;
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    const int row = rg + 8 * i;
    S[i] = i < nr ? S0[(size_t)row * d + c0 + col] : 0.f;
    z[i] = (i < nr && (a.o_lin || slice == 0)) ? a.z_in[hs * d + row] : 0.f;
  }
  const size_t tok_stride = (size_t)sh.H_L * d;
  const T* kb = (const T*)a.k_lin + (size_t)b * a.n * tok_stride + (size_t)h * d;
  const T* qb = (const T*)a.q_lin + (size_t)b * a.n * tok_stride + (size_t)h * d;
  const T* vb = (const T*)a.v_lin + (size_t)b * a.n * tok_stride + (size_t)h * d;

  for (int t0 = 0; t0 < a.n; t0 += LR_STAGE) {
    const int tn = min(LR_STAGE, a.n - t0);
    __syncthreads();
    for (int e = tid; e < LR_STAGE * d; e += 256) {
      const int tt = e / d, c = e % d;
      if (tt < tn) {
        fks[tt][c] = phi(ld1<T>(kb + (size_t)(t0 + tt) * tok_stride + c));
        if (a.o_lin) fqs[tt][c] = phi(ld1<T>(qb + (size_t)(t0 + tt) * tok_stride + c));
      }
    }
    for (int e = tid; e < LR_STAGE * LR_COLS; e += 256) {
      const int tt = e / LR_COLS, c = e % LR_COLS;
      if (tt < tn) vs[tt][c] = ld1<T>(vb + (size_t)(t0 + tt) * tok_stride + c0 + c);
    }
    __syncthreads();
    for (int tt = 0; tt < tn; ++tt) {
      const float v = vs[tt][col];
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int i = 0; i < RMAX; ++i) {
        if (i < nr) {
          const int row = rg + 8 * i;
          const float k = fks[tt][row];
          S[i] = fmaf(k, v, S[i]);
          z[i] += k;
          if (a.o_lin) {
            const float q = fqs[tt][row];
            num = fmaf(q, S[i], num);
            den = fmaf(q, z[i], den);
          }
        }
      }
      if (a.o_lin) {
        num = group_sum(num, 8);
        den = group_sum(den, 8);
        if (rg == 0) {
          const int t = t0 + tt;
          a.o_lin[(((size_t)b * a.n + t) * sh.H_L + h) * d + c0 + col] = normalized ? num / den : num;
        }
      }
    }
  }
  float* Sd = a.S + hs * d * d;
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    const int row = rg + 8 * i;
    if (i < nr) Sd[(size_t)row * d + c0 + col] = S[i];
  }
  if (slice == 0 && col == 0) {
#pragma unroll
    for (int i = 0; i < RMAX; ++i)
      if (i < nr) a.z_out[hs * d + rg + 8 * i] = z[i];
  }
}

hipError_t launch_linear_recurrent(const LinearArgs& a, hipStream_t st) {
  const int slices = a.sh.d / LR_COLS;
  const dim3 grid((unsigned)(a.sh.B * a.sh.H_L * slices));
  if (a.sh.dtype == 0)
    klaunch(k_linear_recurrent<float>, grid, dim3(256), 0, st, a);
  else
    klaunch(k_linear_recurrent<bf16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ void k_copy_f32(float* dst, const float* src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  klaunch(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

}  // namespace lisa
