// Exact per-row top-M selection shared by the select kernel and the fused
// decode kernels ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2).
#pragma once
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

constexpr int NBINS_LOG = 11;
constexpr int NBINS = 1 << NBINS_LOG;
constexpr int SEL_CAND_MAX = 1024;  // boundary-set size resolved by exact ranking

__device__ __forceinline__ int bitlen(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

template <int NW>
struct SelShared {
  uint32_t hist[NBINS];
  alignas(16) uint32_t wa[NW];
  alignas(16) uint32_t wb[NW];
  uint32_t found_bin, found_need, found_cnt, cand_n;
  uint64_t thr;
  uint64_t cand[SEL_CAND_MAX];
  uint32_t gtot[256];  // selected count of every 256-position group
};

// Block-wide min of a and max of b (uniform results): one LDS slot per
// wave, then every wave reduces the NW slots with lane-parallel reads.
// TRAIL: end with a barrier, so that the slots may be rewritten at once
// (without it, the caller must pass a barrier before sm.wa or sm.wb is
// written again).
template <int NW, bool TRAIL = true>
__device__ __forceinline__ void block_min_max(SelShared<NW>& sm, uint32_t a, uint32_t b, uint32_t& mn,
                                              uint32_t& mx) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  a = wave_min_u32(a);
  b = wave_max_u32(b);
  if (lane == 0) {
    sm.wa[wave] = a;
    sm.wb[wave] = b;
  }
  __syncthreads();
  mn = wave_min_u32(sm.wa[lane % NW]);
  mx = wave_max_u32(sm.wb[lane % NW]);
  if constexpr (TRAIL) __syncthreads();
}

// Block-wide inclusive prefix sum in thread order, and the block total.
// TRAIL as for block_min_max (for sm.wa).
template <int NW, bool TRAIL = true>
__device__ __forceinline__ uint32_t block_incl_scan(SelShared<NW>& sm, uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == WAVE - 1) sm.wa[wave] = inc;
  __syncthreads();
  const uint32_t wi = wave_incl_scan_u32(lane < NW ? sm.wa[lane] : 0u);  // prefix over wave totals
  const uint32_t all = rl(wi, NW - 1);
  const uint32_t before = wave == 0 ? 0u : __builtin_amdgcn_readlane((int)wi, wave - 1);
  if constexpr (TRAIL) __syncthreads();
  total = all;
  return before + inc;
}

// Find the bin holding the need-th largest element (bins counted from the
// top).  Thread t owns the NBINS / THREADS consecutive bins from t * that.
// TRAIL: end with a barrier (without it, the caller must pass a barrier
// before sm.found_*, sm.wa or sm.hist is written again).
template <int THREADS, bool TRAIL = true>
__device__ __forceinline__ void find_bin(SelShared<THREADS / WAVE>& sm, uint32_t need, uint32_t& bin,
                                         uint32_t& need_in, uint32_t& cnt) {
  constexpr int BPT = NBINS / THREADS;
  const int tid = threadIdx.x;
  uint32_t h[BPT];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = sm.hist[tid * BPT + i];
    tot += h[i];
  }
  uint32_t all;
  // the barrier below (found_*) also orders the scan's reads of sm.wa
  const uint32_t inc = block_incl_scan<THREADS / WAVE, TRAIL>(sm, tot, all);
  uint32_t above = all - inc;  // elements in bins of higher threads
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (above < need && need <= above + h[i]) {
      sm.found_bin = tid * BPT + i;
      sm.found_need = need - above;
      sm.found_cnt = h[i];
    }
    above += h[i];
  }
  __syncthreads();
  bin = sm.found_bin;
  need_in = sm.found_need;
  cnt = sm.found_cnt;
  if constexpr (TRAIL) __syncthreads();
}

// Keys of the row: in LDS when the row fits (LKEYS), else recomputed from
// the score row in global memory (L2-resident after the first read).
template <int THREADS, int ITEMS, bool LKEYS>
struct KeyStore {
  uint32_t k[LKEYS ? THREADS * ITEMS : 1];
};

// Position layout.  Item i of a thread is element i % 4 of its float4 group
// k = i / 4; group k of lane l in wave w covers positions 4 f .. 4 f + 3 with
// f = (k * NW + w) * 64 + l.  A wave's load of group k is thus 1 KiB of
// consecutive scores (a single CU pulls the row in far faster than with runs
// of positions per thread), and positions ascend with (k, w, l, element).
template <int THREADS>
__device__ __forceinline__ int sel_group(int k) {
  return (k * (THREADS / WAVE) + (int)(threadIdx.x / WAVE)) * WAVE + (int)(threadIdx.x & (WAVE - 1));
}

// Result of select_row for one thread: bit i of `bits` says whether item i
// is selected; rank0[k] is the number of selected positions before group k
// of this lane, i.e. the rank (in ascending position order) of the group's
// first selected position (left unset when the ranks are not asked for).
template <int ITEMS>
struct SelResult {
  uint64_t bits;
  uint32_t rank0[ITEMS / 4];
};

// Exact top-M selection of one score row, by the whole block (every thread
// must call it).  A row of at most M positions is taken whole without
// reading srow.
// The row's scores in the thread's layout (group k of the thread at
// element 4 * sel_group(k)), read before the row length is known: `reach`
// floats from srow are readable (reach >= 1); groups past it re-read the
// last one.  v0 is srow[0].
template <int THREADS, int ITEMS>
struct SelLoad {
  float4 v[ITEMS / 4];
  float v0;
};

template <int THREADS, int ITEMS>
__device__ __forceinline__ void select_load(const float* srow, int reach, SelLoad<THREADS, ITEMS>& ld) {
  const int qmax = (reach - 1) & ~3;  // last 4-aligned group that starts inside the readable part
#pragma unroll
  for (int k = 0; k < ITEMS / 4; ++k)
    ld.v[k] = *reinterpret_cast<const float4*>(srow + min(4 * sel_group<THREADS>(k), qmax));
  ld.v0 = srow[0];
}

template <int THREADS, int ITEMS, bool LKEYS, bool RANKS = true>
__device__ __forceinline__ void select_row(const float* srow, int len, int M, SelShared<THREADS / WAVE>& sm,
                                           KeyStore<THREADS, ITEMS, LKEYS>& ks, const SelLoad<THREADS, ITEMS>& ld,
                                           SelResult<ITEMS>& res) {
  static_assert(ITEMS % 4 == 0 && ITEMS <= 64, "items per thread");
  static_assert(NBINS % THREADS == 0, "bins per thread");
  constexpr int NW = THREADS / WAVE;
  constexpr int K4 = ITEMS / 4;
  static_assert(K4 * NW <= 256, "group totals");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  auto pos_of = [&](int i) -> int { return 4 * sel_group<THREADS>(i >> 2) + (i & 3); };
  uint64_t vmask = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) vmask |= (uint64_t)(pos_of(i) < len) << i;
  if (len <= M) {  // everything is selected: the rank of a position is the position
    res.bits = vmask;
#pragma unroll
    for (int k = 0; k < K4; ++k) res.rank0[k] = (uint32_t)min(4 * sel_group<THREADS>(k), len);
    return;
  }
  float sv[ITEMS];
  {
    const float4* v = ld.v;
    const float fill = ld.v0;  // items past the row end change neither the min nor the max
#pragma unroll
    for (int k = 0; k < K4; ++k) {
      sv[4 * k + 0] = v[k].x; sv[4 * k + 1] = v[k].y; sv[4 * k + 2] = v[k].z; sv[4 * k + 3] = v[k].w;
      if constexpr (LKEYS)
        reinterpret_cast<uint4*>(ks.k)[sel_group<THREADS>(k)] =
            make_uint4(score_key(v[k].x), score_key(v[k].y), score_key(v[k].z), score_key(v[k].w));
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (!((vmask >> i) & 1ull)) sv[i] = fill;
  }
  auto key_at = [&](int i) -> uint32_t {  // key of item i of this thread
    if constexpr (LKEYS) return ks.k[pos_of(i)];
    else return score_key(srow[pos_of(i)]);
  };
  float fmn = sv[0], fmx = sv[0];
#pragma unroll
  for (int k = 1; k < ITEMS; ++k) {
    fmn = fminf(fmn, sv[k]);
    fmx = fmaxf(fmx, sv[k]);
  }
  if (tid == 0) sm.cand_n = 0u;
  uint32_t lo, hi;  // key range of the boundary set
  block_min_max(sm, score_key(fmn), score_key(fmx), lo, hi);

  // Boundary set: elements of value bin bsel (every element without the
  // value pass), narrowed later to keys in [lo, hi] and, once lo == hi,
  // positions in [plo, phi].  Everything above it is selected; `need` of its
  // `cnt` elements are.  `inset` holds this thread's members as bits.
  uint32_t need = (uint32_t)M, cnt = (uint32_t)len;
  uint32_t plo = 0, phi = (uint32_t)(len - 1);
  uint32_t bins[ITEMS];
  uint32_t bsel = 0;
  {
    const float vmin = __uint_as_float((lo & 0x80000000u) ? (lo & 0x7fffffffu) : ~lo);
    const float vmax = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
    const float inv_w = (float)NBINS / (vmax - vmin);
    if (lo != hi && inv_w > 0.f && inv_w < 1e30f) {
#pragma unroll
      for (int i = 0; i < NBINS / THREADS; ++i) sm.hist[tid + i * THREADS] = 0u;
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) bins[k] = min((uint32_t)((sv[k] - vmin) * inv_w), (uint32_t)(NBINS - 1));
      __syncthreads();
#pragma unroll
      for (int k = 0; k < ITEMS; ++k)
        if ((vmask >> k) & 1ull) atomicAdd(&sm.hist[bins[k]], 1u);
      __syncthreads();
      find_bin<THREADS>(sm, need, bsel, need, cnt);
    } else {
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) bins[k] = 0u;
    }
  }
  uint64_t inset = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) inset |= (uint64_t)(bins[k] == bsel) << k;
  inset &= vmask;

  bool narrowed = false;  // [lo, hi] / [plo, phi] restrict the boundary set
  uint64_t thr = 0;       // inside bin bsel: selected iff (key << 32 | pos) >= thr
  for (int pass = 0; pass < 8; ++pass) {
    if (cnt == need) {  // the whole boundary set is taken
      thr = narrowed ? (((uint64_t)lo << 32) | (lo == hi ? plo : 0u)) : 0ull;
      break;
    }
    if (cnt <= (uint32_t)SEL_CAND_MAX) {
      // gather the boundary set (one LDS atomic per wave), then rank it
      const uint32_t act = (uint32_t)__builtin_popcountll(inset);
      const uint32_t winc = wave_incl_scan_u32(act);
      uint32_t wbase = 0;
      if (lane == WAVE - 1 && winc) wbase = atomicAdd(&sm.cand_n, winc);
      uint32_t slot = rl(wbase, WAVE - 1) + winc - act;
      for (uint64_t m = inset; m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        sm.cand[slot++] = ((uint64_t)key_at(k) << 32) | (uint32_t)pos_of(k);
      }
      __syncthreads();
      for (uint32_t c = tid; c < cnt; c += THREADS) {
        const uint64_t mine = sm.cand[c];
        uint32_t above = 0;
        uint32_t k = 0;
        for (; k + 8 <= cnt; k += 8) {  // eight LDS reads in flight
          uint64_t x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = sm.cand[k + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) above += x[u] > mine ? 1u : 0u;
        }
        for (; k < cnt; ++k) above += sm.cand[k] > mine ? 1u : 0u;
        if (above == need - 1) sm.thr = mine;
      }
      __syncthreads();
      thr = sm.thr;
      break;
    }
    // a boundary set too large to rank: one more histogram pass over key
    // bits, or over positions once it is a single key value
    if (!narrowed) {  // key range of the boundary bin
      uint32_t bmin = 0xffffffffu, bmax = 0u;
      for (uint64_t m = inset; m; m &= m - 1) {
        const uint32_t kk = key_at(__builtin_ctzll(m));
        bmin = min(bmin, kk);
        bmax = max(bmax, kk);
      }
      block_min_max(sm, bmin, bmax, lo, hi);
      narrowed = true;
    }
    const bool by_pos = lo == hi;
#pragma unroll
    for (int i = 0; i < NBINS / THREADS; ++i) sm.hist[tid + i * THREADS] = 0u;
    __syncthreads();
    const int shift = by_pos ? max(0, bitlen(phi - plo) - NBINS_LOG) : max(0, bitlen(hi - lo) - NBINS_LOG);
    for (uint64_t m = inset; m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const uint32_t pos = (uint32_t)pos_of(k);
      atomicAdd(&sm.hist[by_pos ? (pos - plo) >> shift : (key_at(k) - lo) >> shift], 1u);
    }
    __syncthreads();
    uint32_t bin, need_in, c;
    find_bin<THREADS>(sm, need, bin, need_in, c);
    if (!by_pos) {
      const uint32_t nlo = lo + (bin << shift);
      const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
      hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
      lo = nlo;
    } else {
      const uint32_t nplo = plo + (bin << shift);
      phi = min(phi, nplo + ((1u << shift) - 1u));
      plo = nplo;
    }
    need = need_in;
    cnt = c;
    // keep the members of the narrowed set
    uint64_t keep = 0;
    for (uint64_t m = inset; m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const uint32_t kk = key_at(k), pos = (uint32_t)pos_of(k);
      if (kk >= lo && kk <= hi && (lo != hi || (pos >= plo && pos <= phi))) keep |= 1ull << k;
    }
    inset = keep;
  }

  // selection bits: higher value bins whole, the boundary bin by threshold
  uint64_t selbits = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) selbits |= (uint64_t)(bins[k] > bsel) << k;
  {
    uint64_t bm = 0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) bm |= (uint64_t)(bins[k] == bsel) << k;
    for (bm &= vmask; bm; bm &= bm - 1) {
      const int k = __builtin_ctzll(bm);
      if ((((uint64_t)key_at(k)) << 32 | (uint32_t)pos_of(k)) >= thr) selbits |= 1ull << k;
    }
  }
  selbits &= vmask;
  if constexpr (!RANKS) {  // the caller wants the selection bits only
    __syncthreads();
    res.bits = selbits;
    return;
  }
  // ranks: prefix over lanes inside each 256-position group (ballots and
  // mbcnt), then over the groups in position order (group k * NW + wave)
  uint32_t excl[K4];
#pragma unroll
  for (int k = 0; k < K4; ++k) {
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((selbits >> (4 * k + e)) & 1ull);
      before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, before));
      tot += (uint32_t)__builtin_popcountll(bal);
    }
    excl[k] = before;
    if (lane == 0) sm.gtot[k * NW + wave] = tot;
  }
  __syncthreads();
  {
    // every wave scans the K4 * NW group totals: lane j sums groups
    // [j * GPL, (j + 1) * GPL), then a wave scan gives each lane's base
    constexpr int NG = K4 * NW;
    constexpr int GPL = (NG + WAVE - 1) / WAVE;
    uint32_t gv[GPL];
    uint32_t part = 0;
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      const int gi = lane * GPL + u;
      gv[u] = gi < NG ? sm.gtot[gi] : 0u;
      part += gv[u];
    }
    const uint32_t base = wave_incl_scan_u32(part) - part;
    // exclusive prefix of group gi = base of its lane + the earlier groups of that lane
#pragma unroll
    for (int k = 0; k < K4; ++k) {
      const int gi = k * NW + wave;
      const int owner = gi / GPL, off = gi % GPL;
      uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)base, owner);
#pragma unroll
      for (int u = 0; u < GPL; ++u)
        if (u < off) before += (uint32_t)__builtin_amdgcn_readlane((int)gv[u], owner);
      res.rank0[k] = before + excl[k];
    }
  }
  __syncthreads();  // sm is free for the caller
  res.bits = selbits;
}

// Calls f(rank, position) for every selected item of this thread, in
// ascending position order.
template <int THREADS, int ITEMS, typename F>
__device__ __forceinline__ void for_each_selected(const SelResult<ITEMS>& res, F f) {
#pragma unroll
  for (int k = 0; k < ITEMS / 4; ++k) {
    const uint32_t g = (uint32_t)(res.bits >> (4 * k)) & 0xfu;
    if (!g) continue;
    const int p = 4 * sel_group<THREADS>(k);
    uint32_t rank = res.rank0[k];
    for (uint32_t m = g; m; m &= m - 1) f(rank++, p + __builtin_ctz(m));
  }
}

template <int ITEMS>
struct RunLoad {
  float4 v[ITEMS / 4];
  float v0;  // srow[0]
};

// The thread's run of scores, read before the row length is known: `reach`
// floats from srow are readable (reach >= 1); groups past it re-read the
// last one.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void run_load(const float* srow, int reach, RunLoad<ITEMS>& ld) {
  const int p0 = (int)threadIdx.x * ITEMS;
  const int qmax = (reach - 1) & ~3;
#pragma unroll
  for (int k = 0; k < ITEMS / 4; ++k) ld.v[k] = *reinterpret_cast<const float4*>(srow + min(p0 + 4 * k, qmax));
  ld.v0 = srow[0];
}

// The same selection with thread-contiguous runs: thread tid owns positions
// p0 = tid * ITEMS .. p0 + ITEMS - 1;
// on return bit k of `selbits` says whether position p0 + k is selected and
// `o` is the number of selected positions before p0, which is the rank of
// the thread's first selected position in ascending order.  A row of at most
// M positions is taken whole without reading srow.
template <int THREADS, int ITEMS, bool LKEYS>
__device__ __forceinline__ void select_row_runs(const float* srow, int len, int M, SelShared<THREADS / WAVE>& sm,
                                                KeyStore<THREADS, ITEMS, LKEYS>& ks, const RunLoad<ITEMS>& ld,
                                                uint64_t& selbits_out, uint32_t& o_out, int& p0_out) {
  static_assert(ITEMS % 4 == 0 && ITEMS <= 64, "items per thread");
  static_assert(NBINS % THREADS == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  if (len <= M) {
    const int p0 = tid * ITEMS;
    const int nval = max(0, min(ITEMS, len - p0));
    selbits_out = nval >= 64 ? ~0ull : ((1ull << nval) - 1ull);
    o_out = (uint32_t)min(p0, len);
    p0_out = p0;
    return;
  }
  const int p0 = tid * ITEMS;
  const int nval = max(0, min(ITEMS, len - p0));  // valid items: a prefix of the run
  const uint64_t vmask = nval >= 64 ? ~0ull : ((1ull << nval) - 1ull);
  float sv[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS / 4; ++k) {
    sv[4 * k + 0] = ld.v[k].x; sv[4 * k + 1] = ld.v[k].y; sv[4 * k + 2] = ld.v[k].z; sv[4 * k + 3] = ld.v[k].w;
  }
  // Items past the row end take a valid value of the thread (or of the row)
  // so that they change neither the min nor the max.
  if (nval < ITEMS) {
    const float fill = nval > 0 ? sv[0] : ld.v0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
      if (k >= nval) sv[k] = fill;
  }
  if constexpr (LKEYS) {
#pragma unroll
    for (int k = 0; k < ITEMS / 4; ++k)
      reinterpret_cast<uint4*>(ks.k + p0)[k] = make_uint4(score_key(sv[4 * k]), score_key(sv[4 * k + 1]),
                                                          score_key(sv[4 * k + 2]), score_key(sv[4 * k + 3]));
  }
  auto key_at = [&](int k) -> uint32_t {  // key of item k of this thread (any k)
    if constexpr (LKEYS) return ks.k[p0 + k];
    else return score_key(srow[p0 + k]);
  };
  float fmn = sv[0], fmx = sv[0];
#pragma unroll
  for (int k = 1; k < ITEMS; ++k) {
    fmn = fminf(fmn, sv[k]);
    fmx = fmaxf(fmx, sv[k]);
  }
  if (tid == 0) sm.cand_n = 0u;
  // the histogram is cleared here; the min/max barrier orders it before
  // the histogram pass
#pragma unroll
  for (int i = 0; i < NBINS / THREADS; ++i) sm.hist[tid + i * THREADS] = 0u;
  uint32_t lo, hi;  // key range of the boundary set
  // no trailing barrier: with value bins, the next writes of sm.wa come
  // after the histogram barrier; without, the barrier is taken below
  block_min_max<THREADS / WAVE, false>(sm, score_key(fmn), score_key(fmx), lo, hi);

  // Boundary set: elements of value bin bsel (every element without the
  // value pass), narrowed later to keys in [lo, hi] and, once lo == hi,
  // positions in [plo, phi].  Everything above it is selected; `need` of its
  // `cnt` elements are.  `inset` holds this thread's members as bits.
  uint32_t need = (uint32_t)M, cnt = (uint32_t)len;
  uint32_t plo = 0, phi = (uint32_t)(len - 1);
  uint32_t bins[ITEMS];
  uint32_t bsel = 0;
  {
    const float vmin = __uint_as_float((lo & 0x80000000u) ? (lo & 0x7fffffffu) : ~lo);
    const float vmax = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
    const float inv_w = (float)NBINS / (vmax - vmin);
    if (lo != hi && inv_w > 0.f && inv_w < 1e30f) {
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) bins[k] = min((uint32_t)((sv[k] - vmin) * inv_w), (uint32_t)(NBINS - 1));
#pragma unroll
      for (int k = 0; k < ITEMS; ++k)
        if (k < nval) atomicAdd(&sm.hist[bins[k]], 1u);
      __syncthreads();
      // no trailing barriers: sm.found_*, sm.wa and sm.hist are written
      // again only after later barriers (the boundary gather's, the
      // narrowing histogram's, the final scan's)
      find_bin<THREADS, false>(sm, need, bsel, need, cnt);
    } else {
      __syncthreads();  // the min/max slots are read before they can be rewritten
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) bins[k] = 0u;
    }
  }
  uint64_t inset = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) inset |= (uint64_t)(bins[k] == bsel) << k;
  inset &= vmask;

  bool narrowed = false;  // [lo, hi] / [plo, phi] restrict the boundary set
  uint64_t thr = 0;       // inside bin bsel: selected iff (key << 32 | pos) >= thr
  for (int pass = 0; pass < 8; ++pass) {
    if (cnt == need) {  // the whole boundary set is taken
      thr = narrowed ? (((uint64_t)lo << 32) | (lo == hi ? plo : 0u)) : 0ull;
      break;
    }
    if (cnt <= (uint32_t)SEL_CAND_MAX) {
      // gather the boundary set (one LDS atomic per wave), then rank it
      const uint32_t act = (uint32_t)__builtin_popcountll(inset);
      const uint32_t winc = wave_incl_scan_u32(act);
      uint32_t wbase = 0;
      if (lane == WAVE - 1 && winc) wbase = atomicAdd(&sm.cand_n, winc);
      uint32_t slot = rl(wbase, WAVE - 1) + winc - act;
      for (uint64_t m = inset; m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        sm.cand[slot++] = ((uint64_t)key_at(k) << 32) | (uint32_t)(p0 + k);
      }
      __syncthreads();
      for (uint32_t c = tid; c < cnt; c += THREADS) {
        const uint64_t mine = sm.cand[c];
        uint32_t above = 0;
        uint32_t k = 0;
        for (; k + 8 <= cnt; k += 8) {  // eight LDS reads in flight
          uint64_t x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = sm.cand[k + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) above += x[u] > mine ? 1u : 0u;
        }
        for (; k < cnt; ++k) above += sm.cand[k] > mine ? 1u : 0u;
        if (above == need - 1) sm.thr = mine;
      }
      __syncthreads();
      thr = sm.thr;
      break;
    }
    // a boundary set too large to rank: one more histogram pass over key
    // bits, or over positions once it is a single key value
    if (!narrowed) {  // key range of the boundary bin
      uint32_t bmin = 0xffffffffu, bmax = 0u;
      for (uint64_t m = inset; m; m &= m - 1) {
        const uint32_t kk = key_at(__builtin_ctzll(m));
        bmin = min(bmin, kk);
        bmax = max(bmax, kk);
      }
      block_min_max(sm, bmin, bmax, lo, hi);
      narrowed = true;
    }
    const bool by_pos = lo == hi;
#pragma unroll
    for (int i = 0; i < NBINS / THREADS; ++i) sm.hist[tid + i * THREADS] = 0u;
    __syncthreads();
    const int shift = by_pos ? max(0, bitlen(phi - plo) - NBINS_LOG) : max(0, bitlen(hi - lo) - NBINS_LOG);
    for (uint64_t m = inset; m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const uint32_t pos = (uint32_t)(p0 + k);
      atomicAdd(&sm.hist[by_pos ? (pos - plo) >> shift : (key_at(k) - lo) >> shift], 1u);
    }
    __syncthreads();
    uint32_t bin, need_in, c;
    find_bin<THREADS>(sm, need, bin, need_in, c);
    if (!by_pos) {
      const uint32_t nlo = lo + (bin << shift);
      const uint64_t top = (uint64_t)nlo + ((1ull << shift) - 1ull);
      hi = (uint32_t)(top < (uint64_t)hi ? top : (uint64_t)hi);
      lo = nlo;
    } else {
      const uint32_t nplo = plo + (bin << shift);
      phi = min(phi, nplo + ((1u << shift) - 1u));
      plo = nplo;
    }
    need = need_in;
    cnt = c;
    // keep the members of the narrowed set
    uint64_t keep = 0;
    for (uint64_t m = inset; m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const uint32_t kk = key_at(k), pos = (uint32_t)(p0 + k);
      if (kk >= lo && kk <= hi && (lo != hi || (pos >= plo && pos <= phi))) keep |= 1ull << k;
    }
    inset = keep;
  }

  // selection bits: higher value bins whole, the boundary bin by threshold
  uint64_t selbits = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) selbits |= (uint64_t)(bins[k] > bsel) << k;
  {
    uint64_t bm = 0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) bm |= (uint64_t)(bins[k] == bsel) << k;
    for (bm &= vmask; bm; bm &= bm - 1) {
      const int k = __builtin_ctzll(bm);
      if ((((uint64_t)key_at(k)) << 32 | (uint32_t)(p0 + k)) >= thr) selbits |= 1ull << k;
    }
  }
  selbits &= vmask;
  const uint32_t nsel = (uint32_t)__builtin_popcountll(selbits);
  uint32_t total;
  // no trailing barrier: the callers write no shared selection state
  // before their own barrier
  uint32_t o = block_incl_scan<THREADS / WAVE, false>(sm, nsel, total) - nsel;
  selbits_out = selbits;
  o_out = o;
  p0_out = p0;
}

}  // namespace lisa
