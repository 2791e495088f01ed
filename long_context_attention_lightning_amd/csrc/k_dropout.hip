// Indexer candidate dropout ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2:
// early in training the top 1.2 M candidates are taken, a random 20% of them
// is masked out, and the sparse attention is filled from the rest, the ratio
// being lowered as training goes on).  Per score row:
//   1. the top n_cand positions (the library's select, as a bitmask);
//   2. k_dropout_compact: the survivors (candidates whose caller-drawn
//      uniform u is at least p), in position order, as a short row of their
//      scores and positions, with its length;
//   3. the top-M select of each short row (ties go to the later entry, which
//      is the later position);
//   4. k_dropout_gather: the selected entries' positions, ascending, -1 padded.
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

__device__ __forceinline__ int dropout_row_len(const DropoutArgs& a, int r) {
  return a.prefill ? r % a.rows_per_seq + 1 : a.seq_lens[r];
}

// One block per row; thread k takes a contiguous run of mask words (at most
// DR_MAXW), so the survivors come out in position order after one block scan
// of the counts.  A word's 32 uniforms and, if any candidate survives, its
// 32 scores are read as independent 16-byte vectors, and the survivor bits
// stay in registers between the counting and the writing pass.
constexpr int DR_MAXW = 8;  // 2048 words of the longest row (65536) over 256 threads

// 32 floats of a row from position 32 w, the part at or past ld read as 0
__device__ __forceinline__ void load_word(const float* row, int64_t ld, int w, float (&v)[32]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t p = 32 * (int64_t)w + 4 * k;
    const float4 x = p < ld ? *reinterpret_cast<const float4*>(row + p) : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * k] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
  }
}

__global__ __launch_bounds__(256) void k_dropout_compact(DropoutArgs a) {
  __shared__ uint32_t wsum[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int len = dropout_row_len(a, r);
  const int words = (len + 31) / 32;
  const int per = (words + 255) / 256, w0 = min(tid * per, words), w1 = min(w0 + per, words);
  const uint32_t* mrow = a.mask + (size_t)r * a.mask_ld;
  const float* urow = a.u + (size_t)r * a.ld;
  uint32_t keep[DR_MAXW];
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < DR_MAXW; ++i) {
    keep[i] = 0u;
    const int w = w0 + i;
    if (w >= w1) continue;
    uint32_t m = mrow[w];
    if (32 * w + 32 > len) m &= (1u << (len - 32 * w)) - 1u;  // len - 32 w < 32 here
    if (!m) continue;
    float u[32];
    load_word(urow, a.ld, w, u);
#pragma unroll
    for (int b = 0; b < 32; ++b) keep[i] |= (((m >> b) & 1u) && u[b] >= a.p) ? (1u << b) : 0u;
    cnt += (uint32_t)__builtin_popcount(keep[i]);
  }
  const uint32_t incl = wave_incl_scan_u32(cnt);
  if (lane == WAVE - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t o = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) o += wsum[w];
    total += wsum[w];
  }
  const float* srow = a.scores + (size_t)r * a.ld;
  float* cs = a.cscore + (size_t)r * a.cld;
  int32_t* cp = a.cpos + (size_t)r * a.cld;
#pragma unroll
  for (int i = 0; i < DR_MAXW; ++i) {
    if (!keep[i]) continue;
    const int w = w0 + i;
    float sv[32];
    load_word(srow, a.ld, w, sv);
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      if ((keep[i] >> b) & 1u) {
        cs[o] = sv[b];
        cp[o] = 32 * w + b;
        ++o;
      }
    }
  }
  if (tid == 0) a.cnt[r] = (int32_t)total;
}

__global__ __launch_bounds__(256) void k_dropout_gather(DropoutArgs a) {
  const int r = blockIdx.x;
  const int32_t* __restrict__ in = a.idx2 + (size_t)r * a.M;
  const int32_t* __restrict__ cp = a.cpos + (size_t)r * a.cld;
  int32_t* __restrict__ out = a.idx_out + (size_t)r * a.M;
  constexpr int U = 8;  // entries per thread in flight
  for (int k0 = threadIdx.x; k0 < a.M; k0 += 256 * U) {
    int e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) e[u] = k0 + 256 * u < a.M ? in[k0 + 256 * u] : -1;
    int p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] = e[u] >= 0 ? cp[e[u]] : -1;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + 256 * u < a.M) out[k0 + 256 * u] = p[u];
  }
}

hipError_t launch_dropout_compact(const DropoutArgs& a, hipStream_t st) {
  klaunch(k_dropout_compact, dim3((unsigned)a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dropout_gather(const DropoutArgs& a, hipStream_t st) {
  klaunch(k_dropout_gather, dim3((unsigned)a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
