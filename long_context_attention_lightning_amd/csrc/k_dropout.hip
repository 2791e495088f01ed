// Indexer candidate dropout ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2:
// early in training the top 1.2 M candidates are taken, a random 20% of them
// is masked out, and the sparse attention is filled from the rest, the ratio
// being lowered as training goes on).  Per score row:
//   1. the top n_cand positions (the library's select, as a bitmask);
//   2. k_dropout_scores: survivors (candidates whose caller-drawn uniform u
//      is at least p) keep their score, every other position gets the
//      lowest float, so
//   3. the top-M select of that row takes the M best survivors, or every
//      survivor and then non-survivors when fewer than M survive;
//   4. k_dropout_filter drops the non-survivors from each ascending list and
//      pads with -1.
// Steps 2 and 4 are elementwise / per-row passes.
#include <float.h>

#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

__device__ __forceinline__ int dropout_row_len(const DropoutArgs& a, int r) {
  return a.prefill ? r % a.rows_per_seq + 1 : a.seq_lens[r];
}

__device__ __forceinline__ bool dropout_survives(const DropoutArgs& a, int r, int p) {
  const uint32_t word = a.mask[(size_t)r * a.mask_ld + (p >> 5)];
  return ((word >> (p & 31)) & 1u) && a.u[(size_t)r * a.ld + p] >= a.p;
}

__global__ __launch_bounds__(256) void k_dropout_scores(DropoutArgs a) {
  const int r = blockIdx.x;
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j >= dropout_row_len(a, r)) return;
  a.s2[(size_t)r * a.ld2 + j] = dropout_survives(a, r, j) ? a.scores[(size_t)r * a.ld + j] : -FLT_MAX;
}

__global__ __launch_bounds__(256) void k_dropout_filter(DropoutArgs a) {
  __shared__ uint32_t wsum[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int M = a.M;
  const int32_t* in = a.idx2 + (size_t)r * M;
  int32_t* out = a.idx_out + (size_t)r * M;
  const int per = (M + 255) / 256, k0 = min(tid * per, M), k1 = min(k0 + per, M);
  auto keep = [&](int k) {
    const int p = in[k];
    return p >= 0 && dropout_survives(a, r, p);
  };
  uint32_t cnt = 0;
  for (int k = k0; k < k1; ++k) cnt += keep(k) ? 1u : 0u;
  const uint32_t incl = wave_incl_scan_u32(cnt);
  if (lane == WAVE - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t o = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) o += wsum[w];
    total += wsum[w];
  }
  for (int k = k0; k < k1; ++k) {  // the chunks are contiguous and in thread order: ascending stays ascending
    const int p = in[k];
    if (p >= 0 && dropout_survives(a, r, p)) out[o++] = p;
  }
  for (int k = (int)total + tid; k < M; k += 256) out[k] = -1;
}

hipError_t launch_dropout_scores(const DropoutArgs& a, int max_len, hipStream_t st) {
  klaunch(k_dropout_scores, dim3((unsigned)a.n_rows, (unsigned)((max_len + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dropout_filter(const DropoutArgs& a, hipStream_t st) {
  klaunch(k_dropout_filter, dim3((unsigned)a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
