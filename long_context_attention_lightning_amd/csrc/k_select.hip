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
#include "lisa_prefill.h"
#include "lisa_select.h"

namespace lisa {
// Row t of sequence b (decode: t = 0).
template <int THREADS, int ITEMS, bool LKEYS>
__device__ __forceinline__ void select_one(const SelectArgs& a, int b, int t, SelShared<THREADS / WAVE>& sm,
                                           KeyStore<THREADS, ITEMS, LKEYS>& ks) {
  const size_t r = (size_t)b * a.rows_per_seq + t;
  const int M = a.M;
  const int tid = threadIdx.x;
  int32_t* orow = a.idx ? a.idx + (size_t)r * a.idx_ld : nullptr;  // null: bitmask only
  uint32_t* mrow = a.mask ? a.mask + (size_t)r * a.mask_ld : nullptr;
  // Decode rows always exist and are read up to max_len while the length is
  // still on its way; prefill rows of at most M positions are not stored
  // (and not read).
  SelLoad<THREADS, ITEMS> ld;
  int len;
  if (a.prefill) {
    len = t + 1;
    if (len > M) select_load<THREADS, ITEMS>(a.scores + ((size_t)b * a.stored_rows + (t - a.first_row)) * a.ld, len, ld);
  } else {
    select_load<THREADS, ITEMS>(a.scores + (size_t)b * a.ld, a.max_len, ld);
    len = a.seq_lens[b];
  }
  const float* srow = a.scores + ((size_t)b * a.stored_rows + (a.prefill ? max(t - a.first_row, 0) : 0)) * a.ld;
  SelResult<ITEMS> res;
  select_row<THREADS, ITEMS, LKEYS>(srow, len, M, sm, ks, ld, res);
  if (orow) for_each_selected<THREADS, ITEMS>(res, [&](uint32_t rank, int pos) { if (rank < (uint32_t)M) orow[rank] = pos; });
  if (mrow) {
    // tiles of 64 keys that hold a selected key of this row (up to 1024 tiles)
    __shared__ uint32_t occ_row[32];
    if (a.occ) {
      if (tid < 32) occ_row[tid] = 0u;
      __syncthreads();
    }
    // eight consecutive lanes hold the 32 positions of one mask word
    const int lane = tid & (WAVE - 1);
#pragma unroll
    for (int k = 0; k < ITEMS / 4; ++k) {
      const int f = sel_group<THREADS>(k);
      uint32_t word = (uint32_t)((res.bits >> (4 * k)) & 0xfull) << (4 * (lane & 7));
      word |= (uint32_t)__shfl_xor((int)word, 1, WAVE);
      word |= (uint32_t)__shfl_xor((int)word, 2, WAVE);
      word |= (uint32_t)__shfl_xor((int)word, 4, WAVE);
      if ((lane & 7) == 0 && 4 * f < len) {
        mrow[f >> 3] = word;
        if (a.occ && word) atomicOr(&occ_row[f >> 9], 1u << ((f >> 4) & 31));  // tile f / 16
      }
    }
    if (a.occ) {  // merge into the row group's occupancy (32 rows share a word)
      __syncthreads();
      uint32_t* orow_occ = a.occ + ((size_t)b * a.occ_rows + t / 32) * a.occ_ld;
      const int words = (len + 2047) / 2048;
      if (tid < words && occ_row[tid]) atomicOr(&orow_occ[tid], occ_row[tid]);
    }
  }
  const int m = M < len ? M : len;
  if (orow)
    for (int k = m + tid; k < M; k += THREADS) orow[k] = -1;
}

template <int THREADS, int ITEMS, bool LKEYS>
__global__ __launch_bounds__(THREADS) void k_select(SelectArgs a) {
  __shared__ SelShared<THREADS / WAVE> sm;
  __shared__ KeyStore<THREADS, ITEMS, LKEYS> ks;
  const int r = blockIdx.x;
  select_one<THREADS, ITEMS, LKEYS>(a, r / a.rows_per_seq, r % a.rows_per_seq, sm, ks);
}

// Many rows of up to 256 * 64 positions (prefill rows, or a large batch of
// decode rows): 256 threads per row, with 16, 32 or 64 scores per thread
// chosen per row by its length (the work of a row scales with the items per
// thread, not with its length); prefill rows go longest first so that the
// short ones fill the tail of the launch.  Keys are recomputed from the
// score row, so the block holds only the histogram and several blocks share
// a CU.
__global__ __launch_bounds__(256) void k_select_rows256(SelectArgs a) {
  __shared__ SelShared<256 / WAVE> sm;
  __shared__ KeyStore<256, 16, false> ks16;
  __shared__ KeyStore<256, 32, false> ks32;
  __shared__ KeyStore<256, 64, false> ks64;
  int b, t, len;
  if (a.prefill) {
    const int n = a.rows_per_seq;
    b = blockIdx.x / n;
    t = n - 1 - (int)(blockIdx.x % n);
    len = t + 1;
  } else {
    b = blockIdx.x;
    t = 0;
    len = a.seq_lens[b];
  }
  if (len <= 256 * 16) select_one<256, 16, false>(a, b, t, sm, ks16);
  else if (len <= 256 * 32) select_one<256, 32, false>(a, b, t, sm, ks32);
  else select_one<256, 64, false>(a, b, t, sm, ks64);
}

// Sliding-window index lists ([LISA] Section 3.2 Stage 1): row t gets the
// min(M, t+1) positions ending at t, ascending, then -1.
__global__ __launch_bounds__(256) void k_window_index(int32_t* idx, int n, int M) {
  const int r = blockIdx.x;  // (sequence, row)
  const int t = r % n;
  const int m = min(M, t + 1);
  for (int k = threadIdx.x; k < M; k += 256) idx[(size_t)r * M + k] = k < m ? t + 1 - m + k : -1;
}

hipError_t launch_window_index(int32_t* idx, int B, int n, int M, hipStream_t st) {
  if (B <= 0 || n <= 0) return hipSuccess;
  klaunch(k_window_index, dim3((unsigned)((size_t)B * n)), dim3(256), 0, st, idx, n, M);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// A kernel rather than a memset, so that the clear is an ordinary kernel
// node when the call is captured into a graph.
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  klaunch(k_zero_u32, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows);
  // one 1024-thread block per row while the rows do not fill the chip
  const bool many = a.prefill || a.n_rows >= 512;
  if (many && a.max_len > 256 * 16 && a.max_len <= 256 * 64) klaunch(k_select_rows256, grid, dim3(256), 0, st, a);
  else if (a.max_len <= 256 * 16) klaunch((k_select<256, 16, true>), grid, dim3(256), 0, st, a);
  else if (a.max_len <= 1024 * 16) klaunch((k_select<1024, 16, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 32) klaunch((k_select<1024, 32, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 64) klaunch((k_select<1024, 64, false>), grid, dim3(1024), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lisa
