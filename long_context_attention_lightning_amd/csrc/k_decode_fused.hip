// Fused top-M selection and gathered attention for decode steps
// ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2: each query keeps the M
// cached positions that score highest under the indexer, its heads' scores
// added, and softmax attention runs over those rows only).
//
// A separate select kernel runs one block per row: one CU has to pull the
// whole score row in, at the rate its own memory parallelism allows, and the
// gather kernel after it waits for another launch and for the index list to
// travel through memory.  Here every (sequence, KV head, split) block selects
// the whole row itself.  The selection is exact and deterministic, so all
// blocks of a row agree.  Each block keeps the positions of its own split of
// the ascending selection in LDS and gathers them right away; the blocks of a
// row read the same score row concurrently from the shared caches.  Each
// block writes its own slice of the index list (KV head 0), so no block
// writes the whole list.  The launch is used while its blocks fit one per CU
// (with 64-position splits for a few sequences, with wide splits of up to
// 2048 positions for batches of tens of sequences).
#include <type_traits>

#include "lisa_attend.h"
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_select.h"

namespace lisa {

constexpr int FS_THREADS = 512;  // 8 waves: 256 registers per lane, no spills
constexpr int FS_MAX_SPLIT = 64;  // positions per split: two attending waves of 32
// Wide splits (bf16, head dim 128): up to 2048 positions, every wave attends
// (32 entries per wave and round), for launches that would need more than one
// block per CU with 64-position splits.
constexpr int FS_WIDE_SPLIT = 2048;

// The values the block needs first come as leading scalar arguments, which
// the compiler lets the hardware preload into SGPRs at wave launch (the
// structs after them are read from the kernel-argument segment, a memory
// round trip, while the score row is already on its way).
template <typename T, int D, int GT, int ITEMS, int MAXS>
__global__ __launch_bounds__(FS_THREADS) void k_select_attend(const float* scores, int64_t sld, const int32_t* seq_lens,
                                                              int max_len, int nsplit, int H_kv, AttnArgs a,
                                                              SelectArgs sa) {
  constexpr int NW = FS_THREADS / WAVE;
  constexpr bool MF = sizeof(T) == 2;  // bf16: MFMA split attention
  // splits of at most MAXS entries: MAXS / 32 attending waves of 32 (all
  // eight for wide splits, which take several rounds)
  constexpr int NWA = MAXS / 32 < NW ? MAXS / 32 : NW;
  static_assert(MAXS <= FS_MAX_SPLIT || MF, "wide splits attend on MFMA");
  using AttT = typename std::conditional<MF, AttnMfmaShared<D, GT, NWA>, AttnMergeShared<NW, GT, D>>::type;
  struct SelPart {
    SelShared<NW> sm;
    KeyStore<FS_THREADS, ITEMS, true> ks;
  };
  // the key store takes more than half of a CU's 160 KB for rows of 16K or
  // more, so the few blocks of a launch spread one per CU
  union Shared {
    SelPart sel;
    AttT att;  // used only after the selection is complete
  };
  __shared__ Shared u;
  __shared__ int plist[MAXS];

  const Shape& sh = a.sh;
  int blk = blockIdx.x;
  const int s = blk % nsplit;
  blk /= nsplit;
  const int g = blk % H_kv;
  const int b = blk / H_kv;  // decode: one row per sequence
  // the score row is read up to max_len while the sequence length loads
  const float* srow = scores + (size_t)b * sld;
  RunLoad<ITEMS> ld;
  run_load<FS_THREADS, ITEMS>(srow, max_len, ld);
  const int len = seq_lens[b];
  const int M = sh.M;
  const int m = min(M, len);
  const int i0 = s * a.split_len;
  if (i0 >= m) return;  // empty split: the combine skips it (the split-0 block pads the index list)
  const int i1 = min(m, i0 + a.split_len);

  // thread-contiguous runs: their compaction is one scan, which is what a
  // latency-bound single row wants
  uint64_t selbits;
  uint32_t o;
  int p0;
  select_row_runs<FS_THREADS, ITEMS, true>(srow, len, M, u.sel.sm, u.sel.ks, ld, selbits, o, p0);

  // this split's positions, and its slice of the index list (KV head 0)
  int32_t* orow = (sa.idx && g == 0) ? sa.idx + (size_t)b * sa.idx_ld : nullptr;
  for (uint64_t mm = selbits; mm; mm &= mm - 1) {
    const int rank = (int)o++;
    if (rank >= i1) break;
    if (rank >= i0) {
      const int pos = p0 + __builtin_ctzll(mm);
      plist[rank - i0] = pos;
      if (orow) orow[rank] = pos;
    }
  }
  if (orow && s == 0)
    for (int k = m + (int)threadIdx.x; k < M; k += FS_THREADS) orow[k] = -1;
  __syncthreads();
  auto pos_of = [&](int i) { return plist[i - i0]; };
  if constexpr (MF) attend_split_mfma<D, GT, FS_THREADS, NWA>(a, b, g, s, len, i0, i1, pos_of, u.att);
  else attend_split<T, D, GT, FS_THREADS, 2>(a, b, g, s, len, i0, i1, pos_of, u.att);
}

#define FS_LEAD (const float*)sa.scores, (int64_t)sa.ld, (const int32_t*)a.seq_lens, sa.max_len, a.nsplit, a.sh.H_kv

template <typename T, int D, int ITEMS, int MAXS>
static hipError_t launch_fs_tdi(const AttnArgs& a, const SelectArgs& sa, dim3 grid, hipStream_t st) {
  const int G = a.sh.H_q / a.sh.H_kv;
  if (G <= 2) klaunch((k_select_attend<T, D, 2, ITEMS, MAXS>), grid, dim3(FS_THREADS), 0, st, FS_LEAD, a, sa);
  else if (G <= 4) klaunch((k_select_attend<T, D, 4, ITEMS, MAXS>), grid, dim3(FS_THREADS), 0, st, FS_LEAD, a, sa);
  else if (G <= 5) klaunch((k_select_attend<T, D, 5, ITEMS, MAXS>), grid, dim3(FS_THREADS), 0, st, FS_LEAD, a, sa);
  else if (G <= 7) klaunch((k_select_attend<T, D, 7, ITEMS, MAXS>), grid, dim3(FS_THREADS), 0, st, FS_LEAD, a, sa);
  else klaunch((k_select_attend<T, D, 8, ITEMS, MAXS>), grid, dim3(FS_THREADS), 0, st, FS_LEAD, a, sa);
  return hipGetLastError();
}
#undef FS_LEAD

template <typename T, int D>
static hipError_t launch_fs_td(const AttnArgs& a, const SelectArgs& sa, dim3 grid, hipStream_t st) {
  if (a.split_len > FS_MAX_SPLIT) {
    if constexpr (sizeof(T) == 2 && D == 128) {
      if (sa.max_len <= FS_THREADS * 32) return launch_fs_tdi<T, D, 32, FS_WIDE_SPLIT>(a, sa, grid, st);
      return launch_fs_tdi<T, D, 64, FS_WIDE_SPLIT>(a, sa, grid, st);
    }
    return hipErrorInvalidValue;
  }
  if (sa.max_len <= FS_THREADS * 32) return launch_fs_tdi<T, D, 32, FS_MAX_SPLIT>(a, sa, grid, st);
  return launch_fs_tdi<T, D, 64, FS_MAX_SPLIT>(a, sa, grid, st);
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

// Selection alone with the same core as k_select_attend, one block per
// decode row, writing the whole index list.
template <int ITEMS>
__global__ __launch_bounds__(FS_THREADS) void k_select_runs(SelectArgs sa) {
  struct Shared {
    SelShared<FS_THREADS / WAVE> sm;
    KeyStore<FS_THREADS, ITEMS, true> ks;
  };
  __shared__ Shared u;
  const int b = blockIdx.x;
  const float* srow = sa.scores + (size_t)b * sa.ld;
  RunLoad<ITEMS> ld;
  run_load<FS_THREADS, ITEMS>(srow, sa.max_len, ld);
  const int len = sa.seq_lens[b];
  const int M = sa.M;
  uint64_t selbits;
  uint32_t o;
  int p0;
  select_row_runs<FS_THREADS, ITEMS, true>(srow, len, M, u.sm, u.ks, ld, selbits, o, p0);
  int32_t* orow = sa.idx + (size_t)b * sa.idx_ld;
  for (uint64_t mm = selbits; mm; mm &= mm - 1) {
    if (o < (uint32_t)M) orow[o] = p0 + __builtin_ctzll(mm);
    ++o;
  }
  for (int k = min(M, len) + (int)threadIdx.x; k < M; k += FS_THREADS) orow[k] = -1;
}

hipError_t launch_select_runs(const SelectArgs& sa, hipStream_t st) {
  if (sa.n_rows <= 0) return hipSuccess;
  if (sa.prefill || !sa.idx) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sa.n_rows);
  if (sa.max_len <= FS_THREADS * 32) klaunch(k_select_runs<32>, grid, dim3(FS_THREADS), 0, st, sa);
  else if (sa.max_len <= FS_THREADS * 64) klaunch(k_select_runs<64>, grid, dim3(FS_THREADS), 0, st, sa);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Every block of the fused launch selects its whole row, and its LDS (the
// key store alone is 64 KB) holds it to one block per CU, so the launch pays
// off only while all its blocks run at once: at most one per CU of the
// MI355X (256).  A second wave of blocks would repeat the select; the
// separate select and gather launches take over there.
constexpr size_t FS_MAX_BLOCKS = 256;

bool select_attend_supported(const Shape& sh, int nsplit, int split_len) {
  const bool wide_ok = sh.dtype != 0 && sh.d == 128 && split_len <= FS_WIDE_SPLIT;
  return sh.max_len <= FS_THREADS * 64 && (split_len <= FS_MAX_SPLIT || wide_ok) && nsplit <= AT_MAX_SPLITS &&
         (size_t)sh.B * sh.H_kv * nsplit <= FS_MAX_BLOCKS;
}

int select_attend_wide_split(const Shape& sh, int positions) {
  for (int sl = 2 * FS_MAX_SPLIT; sl <= FS_WIDE_SPLIT; sl *= 2) {
    const int ns = (positions + sl - 1) / sl;
    if (select_attend_supported(sh, ns, sl)) return sl;
  }
  return 0;
}

hipError_t launch_select_attend(const AttnArgs& a, const SelectArgs& sa, hipStream_t st) {
  return a.sh.dtype == 0 ? launch_fs_t<float>(a, sa, st) : launch_fs_t<bf16_t>(a, sa, st);
}

}  // namespace lisa
