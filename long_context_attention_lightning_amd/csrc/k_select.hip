// Top-M selection of indexer score rows ("LISA", arXiv 2607.19358v1,
// Section 3.2 Stage 2: the M positions with the largest summed score).
//
// One 1024-thread block per row.  Each score becomes a 32-bit
// order-preserving key; appending the position below it gives a composite key
// that is unique per row, so "the M largest composites" is exactly "largest
// score first, later position first on ties".  A most-significant-digit radix
// select (8-bit digits, histograms in LDS) narrows the composite prefix until
// the digit bin at the boundary is taken whole; the keys stay in registers.
// The selected positions are then written in ascending order with a
// block-wide prefix count of ballots, and optionally as a bitmask.
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int ITEMS>
__global__ __launch_bounds__(SEL_THREADS) void k_select(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t found_bin, found_need, found_cnt;
  __shared__ uint32_t wcnt[ITEMS * SEL_WAVES];
  __shared__ uint32_t wsum[SEL_WAVES];

  const int r = blockIdx.x;
  const int b = r / a.rows_per_seq, t = r % a.rows_per_seq;
  const int len = a.prefill ? t + 1 : a.seq_lens[b];
  const int M = a.M;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  int32_t* orow = a.idx + (size_t)r * a.idx_ld;
  uint32_t* mrow = a.mask ? a.mask + (size_t)r * a.mask_ld : nullptr;

  if (len <= M) {  // the whole prefix is selected
    for (int i = tid; i < M; i += SEL_THREADS) orow[i] = i < len ? i : -1;
    if (mrow) {
      const int words = (len + 31) / 32;
      for (int w = tid; w < words; w += SEL_THREADS) {
        const int rem = len - w * 32;
        mrow[w] = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
      }
    }
    return;
  }

  const float* srow = a.scores + ((size_t)b * a.stored_rows + (a.prefill ? t - a.first_row : 0)) * a.ld;
  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int j = i * SEL_THREADS + tid;
    key[i] = j < len ? score_key(srow[j]) : 0u;
  }
  // composite = key << PB | position, PB = bits of (len-1)
  const int PB = 32 - __builtin_clz((unsigned)(len - 1));
  const int TOT = 32 + PB;
  uint64_t pref = 0;
  int depth = 0;  // bits of the composite fixed so far
  uint32_t need = (uint32_t)M;

  // at most ceil(48 / 8) passes: the composite has at most 32 + 16 bits
  for (int pass = 0; pass < 8; ++pass) {
    const int hi = TOT - depth;
    const int w = hi < 8 ? hi : 8;
    const int lo = hi - w;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int j = i * SEL_THREADS + tid;
      if (j < len) {
        const uint64_t c = ((uint64_t)key[i] << PB) | (uint32_t)j;
        if ((c >> hi) == pref) atomicAdd(&hist[(uint32_t)(c >> lo) & ((1u << w) - 1u)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l..4l+3; find the bin holding the need-th largest
      uint32_t h4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) h4[k] = hist[lane * 4 + k];
      const uint32_t tot = h4[0] + h4[1] + h4[2] + h4[3];
      uint32_t suf = tot;  // inclusive suffix sum over lanes >= l
      for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off, WAVE);
        if (lane + off < WAVE) suf += o;
      }
      uint32_t above = suf - tot;  // keys in bins owned by higher lanes
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        if (above < need && need <= above + h4[k]) {
          found_bin = (uint32_t)(lane * 4 + k);
          found_need = need - above;
          found_cnt = h4[k];
        }
        above += h4[k];
      }
    }
    __syncthreads();
    const uint32_t bin = found_bin;
    need = found_need;
    pref = (pref << w) | bin;
    depth += w;
    if (found_cnt == need) break;
  }
  const int shift = TOT - depth;

  // ascending compaction of the selected positions
  uint64_t selbits = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int j = i * SEL_THREADS + tid;
    bool sel = false;
    if (j < len) {
      const uint64_t c = ((uint64_t)key[i] << PB) | (uint32_t)j;
      sel = (c >> shift) >= pref;
    }
    const uint64_t bal = __ballot(sel);
    if (sel) selbits |= (1ull << i);
    if (lane == 0) wcnt[i * SEL_WAVES + wave] = (uint32_t)__builtin_popcountll(bal);
    if (mrow && (lane & 31) == 0) {
      const int word = (i * SEL_THREADS + wave * WAVE + lane) >> 5;
      if (word * 32 < len) mrow[word] = (uint32_t)(bal >> (lane & 32));
    }
  }
  __syncthreads();
  // exclusive scan of wcnt in (i, wave) order = ascending position order
  constexpr int E = ITEMS * SEL_WAVES;
  uint32_t v = tid < E ? wcnt[tid] : 0u;
  uint32_t inc = v;
  for (int off = 1; off < WAVE; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, WAVE);
    if (lane >= off) inc += o;
  }
  if (lane == WAVE - 1) wsum[wave] = inc;
  __syncthreads();
  uint32_t wpre = 0;
  for (int k = 0; k < wave; ++k) wpre += wsum[k];
  __syncthreads();
  if (tid < E) wcnt[tid] = wpre + inc - v;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool sel = (selbits >> i) & 1ull;
    const uint64_t bal = __ballot(sel);
    if (sel) {
      const uint32_t o = wcnt[i * SEL_WAVES + wave] + lanes_below(bal);
      if (o < (uint32_t)M) orow[o] = i * SEL_THREADS + tid;
    }
  }
  const int m = M < len ? M : len;
  for (int k = m + tid; k < M; k += SEL_THREADS) orow[k] = -1;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows), block(SEL_THREADS);
  if (a.max_len <= 1 * SEL_THREADS) hipLaunchKernelGGL(k_select<1>, grid, block, 0, st, a);
  else if (a.max_len <= 4 * SEL_THREADS) hipLaunchKernelGGL(k_select<4>, grid, block, 0, st, a);
  else if (a.max_len <= 16 * SEL_THREADS) hipLaunchKernelGGL(k_select<16>, grid, block, 0, st, a);
  else if (a.max_len <= 32 * SEL_THREADS) hipLaunchKernelGGL(k_select<32>, grid, block, 0, st, a);
  else if (a.max_len <= 64 * SEL_THREADS) hipLaunchKernelGGL(k_select<64>, grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lisa
