// Top-M selection of indexer score rows ("LISA", arXiv 2607.19358v1,
// Section 3.2 Stage 2: the M positions with the largest summed score).
//
// One block per row; each thread keeps the scores of its run of ITEMS
// consecutive positions in registers.  The order is (score descending,
// position descending) with -0.0 equal to +0.0; with the score mapped to an
// order-preserving 32-bit key, the pair (key, position) is unique per row,
// so the selected set is the set of pairs at or above one threshold pair.
//
// A row fits on one CU, whose SIMDs issue about one wave64 instruction per
// cycle in total, so the kernel is built to issue few instructions per score
// and few per wave:
//   1. block min/max of the scores;
//   2. one histogram pass with 2048 LDS bins of equal width in score value
//      between min and max (bin(v) is monotone in v, so every higher bin is
//      taken whole and every lower bin dropped); the boundary bin holds a
//      few elements for realistic score distributions;
//   3. the boundary bin's elements (at most 1024) are gathered and ranked
//      exactly against each other, which gives the threshold pair; a larger
//      boundary set (heavy ties, extreme outliers) gets further histogram
//      passes over key bits and then positions until it is small enough;
//   4. one block scan of per-thread selected counts gives every thread its
//      place in the ascending output; selected positions are written by
//      iterating the set bits of per-thread masks, optionally as a bitmask.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_select.h"

namespace lisa {
template <int THREADS, int ITEMS, bool LKEYS>
__global__ __launch_bounds__(THREADS) void k_select(SelectArgs a) {
  __shared__ SelShared<THREADS / WAVE> sm;
  __shared__ KeyStore<THREADS, ITEMS, LKEYS> ks;
  const int r = blockIdx.x;
  const int b = r / a.rows_per_seq, t = r % a.rows_per_seq;
  const int len = a.prefill ? t + 1 : a.seq_lens[b];
  const int M = a.M;
  const int tid = threadIdx.x;
  int32_t* orow = a.idx ? a.idx + (size_t)r * a.idx_ld : nullptr;  // null: bitmask only
  uint32_t* mrow = a.mask ? a.mask + (size_t)r * a.mask_ld : nullptr;
  // rows of at most M positions have no stored scores (and are not read)
  const float* srow = a.scores + ((size_t)b * a.stored_rows + (a.prefill ? max(t - a.first_row, 0) : 0)) * a.ld;
  uint64_t selbits;
  uint32_t o;
  int p0;
  select_row<THREADS, ITEMS, LKEYS>(srow, len, M, sm, ks, selbits, o, p0);
  if (orow)
    for (uint64_t m = selbits; m; m &= m - 1) {
      if (o < (uint32_t)M) orow[o] = p0 + __builtin_ctzll(m);
      ++o;
    }
  if (mrow) {
    if constexpr (ITEMS >= 32) {
#pragma unroll
      for (int w = 0; w < ITEMS / 32; ++w)
        if (p0 + 32 * w < len) mrow[(p0 >> 5) + w] = (uint32_t)(selbits >> (32 * w));
    } else {
      // 32 / ITEMS threads share a word: OR their shifted bits together
      constexpr int TPW = 32 / ITEMS;
      uint32_t word = (uint32_t)selbits << ((tid % TPW) * ITEMS);
      for (int off = 1; off < TPW; off <<= 1) word |= (uint32_t)__shfl_xor((int)word, off, WAVE);
      if (tid % TPW == 0 && p0 < len) mrow[p0 >> 5] = word;
    }
  }
  const int m = M < len ? M : len;
  if (orow)
    for (int k = m + tid; k < M; k += THREADS) orow[k] = -1;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows);
  if (a.max_len <= 256 * 16) klaunch((k_select<256, 16, true>), grid, dim3(256), 0, st, a);
  else if (a.max_len <= 1024 * 16) klaunch((k_select<1024, 16, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 32) klaunch((k_select<1024, 32, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 64) klaunch((k_select<1024, 64, false>), grid, dim3(1024), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lisa
