// Fused top-M selection and gathered attention for decode steps of a few
// sequences ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2: select the M
// positions with the largest summed indexer score, then softmax attention
// over those cached rows).
//
// With one or a few sequences a separate select kernel runs one block per
// row: one CU has to pull the whole score row in, at the rate its own memory
// parallelism allows, and the gather kernel after it waits for another
// launch and for the index list to travel through memory.  Here every
// (sequence, KV head, split) block selects the whole row itself.  The
// selection is exact and deterministic, so all blocks of a row agree.  Each
// block keeps the positions of its own split of the ascending selection in
// LDS and gathers them right away; the blocks of a row read the same score
// row concurrently from the shared caches.
#include <type_traits>

#include "lisa_attend.h"
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_select.h"

namespace lisa {

constexpr int FS_THREADS = 512;  // 8 waves: 256 registers per lane, no spills
constexpr int FS_MAX_SPLIT = 64;  // positions per split

template <typename T, int D, int GT, int ITEMS>
__global__ __launch_bounds__(FS_THREADS) void k_select_attend(AttnArgs a, SelectArgs sa) {
  constexpr int NW = FS_THREADS / WAVE;
  struct SelPart {
    SelShared<NW> sm;
    KeyStore<FS_THREADS, ITEMS, true> ks;
  };
  constexpr bool MF = sizeof(T) == 2;  // bf16: MFMA split attention
  // splits of at most FS_MAX_SPLIT entries: two attending waves of 32
  using AttT = typename std::conditional<MF, AttnMfmaShared<D, GT, FS_MAX_SPLIT / 32>, AttnMergeShared<NW, GT, D>>::type;
  union Shared {
    SelPart sel;
    AttT att;  // used only after the selection is complete
  };
  __shared__ Shared u;
  __shared__ int plist[FS_MAX_SPLIT];

  const Shape& sh = a.sh;
  int blk = blockIdx.x;
  const int s = blk % a.nsplit;
  blk /= a.nsplit;
  const int g = blk % sh.H_kv;
  const int b = blk / sh.H_kv;  // decode: one row per sequence
  // the score row is read up to max_len while the sequence length loads
  RunLoad<ITEMS> ld;
  run_load<FS_THREADS, ITEMS>(sa.scores + (size_t)b * sa.ld, sa.max_len, ld);
  const int len = a.seq_lens[b];
  const int M = sh.M;
  const int m = min(M, len);
  const int i0 = s * a.split_len;
  const bool want_idx = sa.idx && g == 0 && s == 0;
  if (i0 >= m && !want_idx) return;  // empty split: the combine skips it
  const int i1 = min(m, i0 + a.split_len);

  // thread-contiguous runs: their compaction is one scan, which is what a
  // latency-bound single row wants
  uint64_t selbits;
  uint32_t o;
  int p0;
  select_row_runs<FS_THREADS, ITEMS, true>(sa.scores + (size_t)b * sa.ld, len, M, u.sel.sm, u.sel.ks, ld, selbits, o,
                                           p0);

  if (want_idx) {  // the index list, written once per sequence
    int32_t* orow = sa.idx + (size_t)b * sa.idx_ld;
    uint32_t oo = o;
    for (uint64_t mm = selbits; mm; mm &= mm - 1) {
      if (oo < (uint32_t)M) orow[oo] = p0 + __builtin_ctzll(mm);
      ++oo;
    }
    for (int k = m + (int)threadIdx.x; k < M; k += FS_THREADS) orow[k] = -1;
    if (i0 >= m) return;
  }
  for (uint64_t mm = selbits; mm; mm &= mm - 1) {
    const int rank = (int)o++;
    if (rank >= i1) break;
    if (rank >= i0) plist[rank - i0] = p0 + __builtin_ctzll(mm);
  }
  __syncthreads();
  auto pos_of = [&](int i) { return plist[i - i0]; };
  if constexpr (MF) attend_split_mfma<D, GT, FS_THREADS, FS_MAX_SPLIT / 32>(a, b, g, s, len, i0, i1, pos_of, u.att);
  else attend_split<T, D, GT, FS_THREADS, 2>(a, b, g, s, len, i0, i1, pos_of, u.att);
}

template <typename T, int D, int ITEMS>
static hipError_t launch_fs_tdi(const AttnArgs& a, const SelectArgs& sa, dim3 grid, hipStream_t st) {
  const int G = a.sh.H_q / a.sh.H_kv;
  if (G <= 2) klaunch((k_select_attend<T, D, 2, ITEMS>), grid, dim3(FS_THREADS), 0, st, a, sa);
  else if (G <= 4) klaunch((k_select_attend<T, D, 4, ITEMS>), grid, dim3(FS_THREADS), 0, st, a, sa);
  else if (G <= 5) klaunch((k_select_attend<T, D, 5, ITEMS>), grid, dim3(FS_THREADS), 0, st, a, sa);
  else if (G <= 7) klaunch((k_select_attend<T, D, 7, ITEMS>), grid, dim3(FS_THREADS), 0, st, a, sa);
  else klaunch((k_select_attend<T, D, 8, ITEMS>), grid, dim3(FS_THREADS), 0, st, a, sa);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fs_td(const AttnArgs& a, const SelectArgs& sa, dim3 grid, hipStream_t st) {
  if (sa.max_len <= FS_THREADS * 32) return launch_fs_tdi<T, D, 32>(a, sa, grid, st);
  return launch_fs_tdi<T, D, 64>(a, sa, grid, st);
}

template <typename T>
static hipError_t launch_fs_t(const AttnArgs& a, const SelectArgs& sa, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.sh.B * a.sh.H_kv * a.nsplit));
  switch (a.sh.d) {
    case 32: return launch_fs_td<T, 32>(a, sa, grid, st);
    case 64: return launch_fs_td<T, 64>(a, sa, grid, st);
    case 128: return launch_fs_td<T, 128>(a, sa, grid, st);
    default: return hipErrorInvalidValue;
  }
}

bool select_attend_supported(const Shape& sh, int nsplit, int split_len) {
  return sh.max_len <= FS_THREADS * 64 && split_len <= FS_MAX_SPLIT && nsplit <= AT_MAX_SPLITS &&
         (size_t)sh.B * sh.H_kv * nsplit <= 512;
}

hipError_t launch_select_attend(const AttnArgs& a, const SelectArgs& sa, hipStream_t st) {
  return a.sh.dtype == 0 ? launch_fs_t<float>(a, sa, st) : launch_fs_t<bf16_t>(a, sa, st);
}

}  // namespace lisa
