// Attention coverage of a selection ("LISA", arXiv 2607.19358v1, Section 4,
// "Optimal Window Size M and Attention Coverage", Eq. 10): for one query row
// and query head, the share of its dense causal softmax weight that falls on
// the selected positions, and the share of the head's own M largest weights
// (the bound no shared M-set can exceed).
//
//  1. logits: q_h . k_j / sqrt(d) in fp32 for every key of the row and the G
//     query heads of one KV head per block, so each key row is read once
//     per row (HBM-bound on the key reads).  Each block also leaves, per
//     head, the max of its 256 logits and the sum of exp(logit - max), so
//     the row's softmax normaliser needs no second pass over the logits.
//       bf16: the logits are MFMA tiles [16 keys x 16 heads] (heads past G
//       are zero columns), key rows loaded straight into the A operand and
//       the query heads held as B operands for the whole block.
//       fp32: four lanes share a key, each reading a quarter of the row;
//       query heads come from LDS as broadcasts; a quad sum finishes each
//       dot product.
//  2. top-M of each head's logit row (exp is monotone, so the M largest
//     logits carry the M largest weights), only when the bound is asked for.
//  3. reduce: per (row, head) the blocks' (max, sum) pairs are merged, and
//     exp(logit - max) is summed over the selected and the bound positions.
#include <math.h>

#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"

namespace lisa {

constexpr int MS_KEYS = 256;  // keys per logits block (4 waves x 4 passes x 16 keys)

template <typename T, int D>
__global__ __launch_bounds__(256) void k_mass_logits(MassArgs a) {
  __shared__ float qs[8][D];
  const Shape& sh = a.sh;
  const int r = blockIdx.z, kvh = blockIdx.x;
  const int G = sh.H_q / sh.H_kv;
  const int len = a.row_len[r];
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && tid < G) a.lens[(size_t)r * sh.H_q + kvh * G + tid] = len;
  const int j0 = MS_KEYS * blockIdx.y;
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
  float pm[8], ps[8];  // running (max, sum) per head over this quad's keys
#pragma unroll
  for (int h = 0; h < 8; ++h) { pm[h] = -INFINITY; ps[h] = 0.f; }
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
      const float s = group_sum(acc[h], 4) * scale;  // the four quarters of key j
      if (j < len) {
        if ((h & 3) == kq) lrow[(size_t)h * a.ld + j] = s;
        lse_merge(pm[h], ps[h], s, 1.f);
      }
    }
  }
  // merge the 16 quads of the wave (all four lanes of a quad hold the same
  // pairs), then the four waves
  __shared__ float wm[4][8], wsum[4][8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= G) break;
    lse_merge_xor(pm[h], ps[h], 4);
    lse_merge_xor(pm[h], ps[h], 8);
    lse_merge_xor(pm[h], ps[h], 16);
    lse_merge_xor(pm[h], ps[h], 32);
    if (lane == 0) { wm[wave][h] = pm[h]; wsum[wave][h] = ps[h]; }
  }
  __syncthreads();
  if (tid < G) {
    float m = wm[0][tid], sm = wsum[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(m, sm, wm[w][tid], wsum[w][tid]);
    a.part[((size_t)r * sh.H_q + (size_t)kvh * G + tid) * a.part_ld + blockIdx.y] = make_float2(m, sm);
  }
}

// bf16 logits on MFMA.  Wave w of the block takes keys j0 + 64 w .. + 63 as
// four 16-key tiles; lane (r16, g) loads 16 bytes of key r16's row per
// 32-element step (A operand) and holds query head r16 as B operands, so the
// accumulator gives lane (r16, g) the logits of keys 4 g .. 4 g + 3 of the
// tile for head r16.
template <int D>
__global__ __launch_bounds__(256) void k_mass_logits_mfma(MassArgs a) {
  __shared__ float wm[4][16], wsum[4][16];
  const Shape& sh = a.sh;
  const int r = blockIdx.z, kvh = blockIdx.x;
  const int G = sh.H_q / sh.H_kv;
  const int len = a.row_len[r];
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && tid < G) a.lens[(size_t)r * sh.H_q + kvh * G + tid] = len;
  const int j0 = MS_KEYS * blockIdx.y;
  if (j0 >= len) return;
  const int seq = a.row_seq ? a.row_seq[r] : r;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE, r16 = lane & 15, g = lane >> 4;
  constexpr int KS = D / 32;
  bf16x8 qf[KS];
  {
    const bf16_t* qh = (const bf16_t*)a.q + ((size_t)r * sh.H_q + (size_t)kvh * G + min(r16, G - 1)) * D + 8 * g;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint4 v = ld16(qh + 32 * k);
      if (r16 >= G) v = make_uint4(0u, 0u, 0u, 0u);
      qf[k] = as_bf16x8(v);
    }
  }
  const bf16_t* kbase = (const bf16_t*)a.k_cache + ((size_t)seq * sh.cap * sh.H_kv + kvh) * D + 8 * g;
  const size_t kstride = (size_t)sh.H_kv * D;
  const int jw = j0 + 64 * wave;
  uint4 kf[4][KS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int key = jw + 16 * t + r16;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      kf[t][k] = key < len ? ld16(kbase + (size_t)key * kstride + 32 * k) : make_uint4(0u, 0u, 0u, 0u);
  }
  const float scale = a.scale;
  float v[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = zero4();
#pragma unroll
    for (int k = 0; k < KS; ++k) acc = mfma16(as_bf16x8(kf[t][k]), qf[k], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[t][e] = acc[e] * scale;
  }
  // stores: keys jw + 16 t + 4 g + e of head r16
  float* lrow = a.logits + ((size_t)r * sh.H_q + (size_t)kvh * G + r16) * a.ld;
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k0 = jw + 16 * t + 4 * g;
    if (r16 < G) {
      if (k0 + 3 < len) {
        *reinterpret_cast<float4*>(lrow + k0) = make_float4(v[t][0], v[t][1], v[t][2], v[t][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k0 + e < len) lrow[k0 + e] = v[t][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (k0 + e < len) mx = fmaxf(mx, v[t][e]);
  }
  float sm = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (jw + 16 * t + 4 * g + e < len) sm += expf(v[t][e] - mx);
  }
  lse_merge_xor(mx, sm, 16);  // the four lane groups g of head r16
  lse_merge_xor(mx, sm, 32);
  if (g == 0) { wm[wave][r16] = mx; wsum[wave][r16] = sm; }
  __syncthreads();
  if (tid < G) {
    float m = wm[0][tid], s2 = wsum[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(m, s2, wm[w][tid], wsum[w][tid]);
    a.part[((size_t)r * sh.H_q + (size_t)kvh * G + tid) * a.part_ld + blockIdx.y] = make_float2(m, s2);
  }
}

__global__ __launch_bounds__(256) void k_mass_reduce(MassArgs a) {
  __shared__ float red[4], rm[4], rs[4];
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H_q = a.sh.H_q, M = a.sh.M;
  const int len = a.row_len[r];
  const float* s = a.logits + ((size_t)r * H_q + h) * a.ld;
  // the row's (max, sum of exp) from the logits blocks' pairs
  const int nkb = (len + MS_KEYS - 1) / MS_KEYS;
  const float2* part = a.part + ((size_t)r * H_q + h) * a.part_ld;
  float mx = -INFINITY, z = 0.f;
  for (int k = tid; k < nkb; k += 256) {
    const float2 p = part[k];
    lse_merge(mx, z, p.x, p.y);
  }
#pragma unroll
  for (int mask = 1; mask < WAVE; mask <<= 1) lse_merge_xor(mx, z, mask);
  if ((tid & (WAVE - 1)) == 0) { rm[tid / WAVE] = mx; rs[tid / WAVE] = z; }
  __syncthreads();
  mx = rm[0]; z = rs[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_merge(mx, z, rm[w], rs[w]);
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

int mass_key_blocks(int max_len) { return (max_len + MS_KEYS - 1) / MS_KEYS; }

hipError_t launch_mass_logits(const MassArgs& a, int max_len, hipStream_t st) {
  // KV heads fastest: the blocks that read the H_kv parts of the same key
  // rows are dispatched together
  const dim3 grid((unsigned)a.sh.H_kv, (unsigned)mass_key_blocks(max_len), (unsigned)a.n_rows);
  const bool bf = a.sh.dtype == 1;
  switch (a.sh.d) {
    case 32:
      if (bf) klaunch((k_mass_logits_mfma<32>), grid, dim3(256), 0, st, a);
      else klaunch((k_mass_logits<float, 32>), grid, dim3(256), 0, st, a);
      break;
    case 64:
      if (bf) klaunch((k_mass_logits_mfma<64>), grid, dim3(256), 0, st, a);
      else klaunch((k_mass_logits<float, 64>), grid, dim3(256), 0, st, a);
      break;
    default:
      if (bf) klaunch((k_mass_logits_mfma<128>), grid, dim3(256), 0, st, a);
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
