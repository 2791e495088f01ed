// Top-M selection of indexer score rows ("LISA", arXiv 2607.19358v1,
// Section 3.2 Stage 2: per query, the M positions ranked highest by the
// indexer score summed over its heads).
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
// Row t of sequence b (decode: t = 0).  RANKS: the launch writes index
// lists (a.idx), which need each selected position's rank; without them
// only the selection bitmask is written.
template <int THREADS, int ITEMS, bool LKEYS, bool RANKS = true>
__device__ __forceinline__ void select_one(const SelectArgs& a, int b, int t, SelShared<THREADS / WAVE>& sm,
                                           KeyStore<THREADS, ITEMS, LKEYS>& ks) {
  const size_t r = (size_t)b * a.rows_per_seq + t;
  const int M = a.M;
  const int tid = threadIdx.x;
  int32_t* orow = (RANKS && a.idx) ? a.idx + (size_t)r * a.idx_ld : nullptr;  // null: bitmask only
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
  select_row<THREADS, ITEMS, LKEYS, RANKS>(srow, len, M, sm, ks, ld, res);
  if (orow) for_each_selected<THREADS, ITEMS>(res, [&](uint32_t rank, int pos) { if (rank < (uint32_t)M) orow[rank] = pos; });
  if (mrow) {
    // eight consecutive lanes hold the 32 positions of one mask word
    const int lane = tid & (WAVE - 1);
#pragma unroll
    for (int k = 0; k < ITEMS / 4; ++k) {
      const int f = sel_group<THREADS>(k);
      uint32_t word = (uint32_t)((res.bits >> (4 * k)) & 0xfull) << (4 * (lane & 7));
      word |= (uint32_t)__shfl_xor((int)word, 1, WAVE);
      word |= (uint32_t)__shfl_xor((int)word, 2, WAVE);
      word |= (uint32_t)__shfl_xor((int)word, 4, WAVE);
      if ((lane & 7) == 0 && 4 * f < len) mrow[f >> 3] = word;
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
template <bool RANKS>  // bitmask only: held to 128 registers, four blocks per CU
__global__ __launch_bounds__(256, RANKS ? 1 : 4) void k_select_rows256(SelectArgs a) {
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
  if (len <= 256 * 16) select_one<256, 16, false, RANKS>(a, b, t, sm, ks16);
  else if (len <= 256 * 32) select_one<256, 32, false, RANKS>(a, b, t, sm, ks32);
  else select_one<256, 64, false, RANKS>(a, b, t, sm, ks64);
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

// Key-tile occupancy of a prefill selection bitmask: one block per group of
// 32 query rows of a sequence.  Lane w of a wave ORs mask word w of the 32
// rows (64 consecutive words = 32 tiles of 64 keys per wave pass); a ballot
// turns that into one occupancy word, tile bit t set when word 2 t or
// 2 t + 1 is non-zero in some row.  Rows past n and words past a row's
// length are zero in the bitmask or never read.
__global__ __launch_bounds__(256) void k_mask_occupancy(const uint32_t* mask, int64_t mask_ld, int n, uint32_t* occ,
                                                        int64_t occ_ld) {
  const int groups = (n + 31) / 32;
  const int b = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r0 = 32 * grp, r1 = min(n, r0 + 32);
  const int words = (r1 + 31) / 32;  // mask words any row of the group can use
  const uint32_t* mb = mask + ((size_t)b * n + r0) * mask_ld;
  uint32_t* ob = occ + ((size_t)b * groups + grp) * occ_ld;
  for (int ow = wave; ow < occ_ld; ow += 4) {
    const int w = 64 * ow + lane;
    // the group's 32 rows at once: one memory round trip per occupancy word
    uint32_t v[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = (w < words && r < r1 - r0) ? mb[(size_t)r * mask_ld + w] : 0u;
    uint32_t acc = 0;
#pragma unroll
    for (int r = 0; r < 32; ++r) acc |= v[r];
    uint64_t nz = __builtin_amdgcn_ballot_w64(acc != 0u);
    nz = (nz | (nz >> 1)) & 0x5555555555555555ull;  // bit 2t: tile t occupied; compact to bit t
    nz = (nz | (nz >> 1)) & 0x3333333333333333ull;
    nz = (nz | (nz >> 2)) & 0x0f0f0f0f0f0f0f0full;
    nz = (nz | (nz >> 4)) & 0x00ff00ff00ff00ffull;
    nz = (nz | (nz >> 8)) & 0x0000ffff0000ffffull;
    nz = (nz | (nz >> 16)) & 0x00000000ffffffffull;
    if (lane == 0) ob[ow] = (uint32_t)nz;
  }
}

hipError_t launch_mask_occupancy(const uint32_t* mask, int64_t mask_ld, int B, int n, uint32_t* occ, int64_t occ_ld,
                                 hipStream_t st) {
  if (B <= 0 || n <= 0) return hipSuccess;
  klaunch(k_mask_occupancy, dim3((unsigned)((size_t)B * ((n + 31) / 32))), dim3(256), 0, st, mask, mask_ld, n, occ,
          occ_ld);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows);
  // one 1024-thread block per row while the rows do not fill the chip
  const bool many = a.prefill || a.n_rows >= 512;
  if (many && a.max_len > 256 * 16 && a.max_len <= 256 * 64) {
    if (a.idx) klaunch(k_select_rows256<true>, grid, dim3(256), 0, st, a);
    else klaunch(k_select_rows256<false>, grid, dim3(256), 0, st, a);  // bitmask only
  }
  else if (a.max_len <= 256 * 16) klaunch((k_select<256, 16, true>), grid, dim3(256), 0, st, a);
  else if (a.max_len <= 1024 * 16) klaunch((k_select<1024, 16, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 32) klaunch((k_select<1024, 32, true>), grid, dim3(1024), 0, st, a);
  else if (a.max_len <= 1024 * 64) klaunch((k_select<1024, 64, false>), grid, dim3(1024), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lisa
