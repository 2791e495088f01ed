// Attention coverage of a selection ("LISA", arXiv 2607.19358v1, Section 4,
// "Optimal Window Size M and Attention Coverage", Eq. 10): for one query row
// and query head, the share of its dense causal softmax weight that falls on
// the selected positions, and the share of the head's own M largest weights
// (the bound no shared M-set can exceed).
//
//  1. k_mass_logits: the fp32 logits q_h . k_j / sqrt(d) of every key of the
//     row, for the G query heads of one KV head per block, so each key row
//     is read once per row (HBM-bound on the key reads).  Four lanes share a
//     key: each reads a quarter of the row in 16-byte pieces (64 contiguous
//     bytes per key and load), the query heads come from LDS as broadcasts,
//     and a quad reduction finishes each dot product.
//  2. top-M of each head's logit row (the exp is monotone, so the M largest
//     logits carry the M largest weights), only when the bound is asked for.
//  3. k_mass_reduce: per (row, head) the maximum, the sum of exp(s - max)
//     over the row, and the same sum over the selected and the bound sets.
#include <math.h>

#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

constexpr int MS_KEYS = 256;  // keys per logits block (4 waves x 4 passes x 16 keys)

template <typename T, int D>
__global__ __launch_bounds__(256) void k_mass_logits(MassArgs a) {
  __shared__ float qs[8][D];
  const Shape& sh = a.sh;
  const int r = blockIdx.x, kvh = blockIdx.y;
  const int G = sh.H_q / sh.H_kv;
  const int len = a.row_len[r];
  const int tid = threadIdx.x;
  if (blockIdx.z == 0 && tid < G) a.lens[(size_t)r * sh.H_q + kvh * G + tid] = len;
  const int j0 = MS_KEYS * blockIdx.z;
  if (j0 >= len) return;
  const int seq = a.row_seq ? a.row_seq[r] : r;
  const T* qr = (const T*)a.q + ((size_t)r * sh.H_q + (size_t)kvh * G) * D;
  for (int e = tid; e < G * D; e += 256) qs[e / D][e % D] = ld1(qr + e);
  __syncthreads();

  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int NL = D / (4 * E);         // pieces per lane
  const int lane = tid & (WAVE - 1), wave = tid / WAVE, kq = lane & 3, kr = lane >> 2;
  const T* kb = (const T*)a.k_cache + ((size_t)seq * sh.cap * sh.H_kv + kvh) * D;
  const size_t kstride = (size_t)sh.H_kv * D;
  const float scale = a.scale;
  float* lrow = a.logits + ((size_t)r * sh.H_q + (size_t)kvh * G) * a.ld;
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    const int jb = j0 + 64 * wave + 16 * p;
    if (jb >= len) break;  // wave-uniform
    const int j = jb + kr;
    float acc[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] = 0.f;
    if (j < len) {
      const T* krow = kb + (size_t)j * kstride;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int c = (kq + 4 * i) * E;  // first element of this piece
        float kf[E];
        Vec<T>::unpack(ld16(krow + c), kf);
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          if (h >= G) break;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h] = fmaf(kf[e], qs[h][c + e], acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h >= G) break;
      const float s = group_sum(acc[h], 4);  // the four quarters of key j
      if (j < len && (h & 3) == kq) lrow[(size_t)h * a.ld + j] = s * scale;
    }
  }
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

__global__ __launch_bounds__(256) void k_mass_reduce(MassArgs a) {
  __shared__ float red[4];
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H_q = a.sh.H_q, M = a.sh.M;
  const int len = a.row_len[r];
  const float* s = a.logits + ((size_t)r * H_q + h) * a.ld;
  float mx = -INFINITY;
  for (int j = tid; j < len; j += 256) mx = fmaxf(mx, s[j]);
  mx = block_max256(mx, red);
  float z = 0.f;
  for (int j = tid; j < len; j += 256) z += expf(s[j] - mx);
  z = block_sum256(z, red);
  float num = 0.f;
  const int32_t* sel = a.idx + (size_t)r * M;
  for (int k = tid; k < M; k += 256) {
    const int p = sel[k];
    if (p >= 0 && p < len) num += expf(s[p] - mx);
  }
  num = block_sum256(num, red);
  float bnum = 0.f;
  if (a.bound) {
    const int32_t* bs = a.bidx + ((size_t)r * H_q + h) * M;
    for (int k = tid; k < M; k += 256) {
      const int p = bs[k];
      if (p >= 0) bnum += expf(s[p] - mx);
    }
    bnum = block_sum256(bnum, red);
  }
  if (tid == 0) {
    a.mass[(size_t)r * H_q + h] = num / z;
    if (a.bound) a.bound[(size_t)r * H_q + h] = bnum / z;
  }
}

hipError_t launch_mass_logits(const MassArgs& a, int max_len, hipStream_t st) {
  const dim3 grid((unsigned)a.n_rows, (unsigned)a.sh.H_kv, (unsigned)((max_len + MS_KEYS - 1) / MS_KEYS));
  const bool bf = a.sh.dtype == 1;
  switch (a.sh.d) {
    case 32:
      if (bf) klaunch((k_mass_logits<bf16_t, 32>), grid, dim3(256), 0, st, a);
      else klaunch((k_mass_logits<float, 32>), grid, dim3(256), 0, st, a);
      break;
    case 64:
      if (bf) klaunch((k_mass_logits<bf16_t, 64>), grid, dim3(256), 0, st, a);
      else klaunch((k_mass_logits<float, 64>), grid, dim3(256), 0, st, a);
      break;
    default:
      if (bf) klaunch((k_mass_logits<bf16_t, 128>), grid, dim3(256), 0, st, a);
      else klaunch((k_mass_logits<float, 128>), grid, dim3(256), 0, st, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_mass_reduce(const MassArgs& a, hipStream_t st) {
  klaunch(k_mass_reduce, dim3((unsigned)a.n_rows, (unsigned)a.sh.H_q), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
