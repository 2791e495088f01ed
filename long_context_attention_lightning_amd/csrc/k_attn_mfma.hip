// Sparse GQA attention of the LISA prefill on bf16 MFMA ("LISA", arXiv
// 2607.19358v1, Section 3.2: each query attends, with softmax, to the M
// cached positions its indexer selected; Section 3.3 Eq. 5 and the gate
// g = sigmoid(x W_g) fuse the result with the linear branch).
//
// The selected sets come as one bitmask row per query (bit j of row t set
// when position j is selected).  For uniformly spread selections every
// 64 x 64 tile of the causal triangle holds selected pairs, so gathering
// rows per query would move each K/V row many times over; this kernel
// instead walks the causal key tiles once per block of 64 queries, as a
// flash-attention forward pass, and sends unselected pairs to -inf before
// the online softmax.
//
// Block = 4 waves of one KV head, each wave one (query head, 32 query
// positions) unit; the K and V tiles of 64 keys are staged row-major in LDS
// for all four waves.  Per tile a wave computes S^T = K Q^T (keys along the
// accumulator rows, so a lane holds four consecutive keys of one query),
// masks and exponentiates it, and feeds the probabilities straight from
// registers into O += P V; the V operands come from transposing LDS loads in
// the key order of the P operand.
#include <type_traits>

#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"
#include "lisa_prefill.h"

namespace lisa {

constexpr int AK = 64;    // keys per tile
constexpr int AP = 2;     // query tiles of 16 per wave
constexpr int AQ = 16 * AP;

// Both tiles are stored row-major with rows D + 16 elements apart: 8 dwords
// modulo the 64 LDS banks, and 16-byte aligned.  Measured on gfx950 with the
// access patterns below (16-byte K operand reads of 16 rows per column
// block, transposing 8-byte V reads): this stride runs conflict-free at 4
// LDS cycles per wave-wide 16-byte read, while a stride of 4 dwords modulo
// 64 takes 8 (half of them bank-conflict stalls) and an unaligned one also 8.
// Two buffers: tile kt is read from one while tile kt + 1 is staged into
// the other.
template <int D>
struct AttnShared {
  bf16_t k[2][AK][D + 16];
  bf16_t v[2][AK][D + 16];
};

template <int D>
struct AttnRegs {
  static constexpr int NK = AK * D / 8 / 256;   // 16-byte K (and V) vectors per thread
  uint4 k[NK], v[NK];
  uint2 mw[AP];                                 // mask words of the lane's query rows
};

// Thread tid stages vectors e = tid + 256 m: row e / (D / 8), columns
// 8 (e % (D / 8)) .. + 7, of both tiles.
template <int D>
__device__ __forceinline__ void attn_stage(const AttnRegs<D>& r, AttnShared<D>& sm, int buf, bool with_v) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < AttnRegs<D>::NK; ++m) {
    const int e = tid + 256 * m;
    *reinterpret_cast<uint4*>(&sm.k[buf][e / (D / 8)][8 * (e % (D / 8))]) = r.k[m];
  }
  if (!with_v) return;
#pragma unroll
  for (int m = 0; m < AttnRegs<D>::NK; ++m) {
    const int e = tid + 256 * m;
    *reinterpret_cast<uint4*>(&sm.v[buf][e / (D / 8)][8 * (e % (D / 8))]) = r.v[m];
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// The transposing LDS load (ds_read_b64_tr_b16) works on groups of 16 lanes:
// if lane j of a group points at 4 consecutive 16-bit elements X[j][0..3],
// lane l receives X[4 e + l / 4][l % 4] for e = 0..3.  With lane j pointing
// at row R0 + j / 4, columns C0 + 4 (j % 4) .. + 3 of a row-major tile, lane
// l thus receives rows R0 .. R0 + 3 of column C0 + l: four consecutive keys
// of one V column, the layout of an MFMA B fragment.
__device__ __forceinline__ v4i16 lds_read_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_prefill_mfma(AttnMaskArgs a) {  // two blocks per CU
  __shared__ AttnShared<D> sm;
  __shared__ uint16_t tiles[ATTN_MAX_TILES];  // the key tiles the block walks, ascending
  __shared__ int tile_count[4];
  const Shape& sh = a.sh;
  const int n = a.n;
  const int G = sh.H_q / sh.H_kv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);  // uniform: scalar unit bookkeeping
  const int r16 = lane & 15, g = lane >> 4;
  // Work units are (query tile of AQ rows, head of the KV group) pairs,
  // numbered head-fastest from the last query tile down; block k takes
  // units 4k .. 4k + 3, one per wave (adjacent query tiles: at most two for
  // GQA groups of two or more heads, four for one; the staged K/V tiles
  // serve every wave), longest causal rows first.
  const int nqt = (n + AQ - 1) / AQ;
  const int units = nqt * G;
  const int per = sh.B * sh.H_kv;
  const int kblk = (int)(blockIdx.x / per);
  const int rest = (int)(blockIdx.x % per);
  const int kvh = rest % sh.H_kv, b = rest / sh.H_kv;
  const int unit = 4 * kblk + wave;
  const bool active = unit < units;  // idle waves repeat the last unit and store nothing
  const int uu = min(unit, units - 1);
  const int h = kvh * G + uu % G;
  const int T0 = (nqt - 1 - uu / G) * AQ;
  // keys up to the last row of the block's highest query tile
  const int tmax = min((nqt - (4 * kblk) / G) * AQ, n) - 1;
  // sliding window: key tiles before the window of the block's lowest row
  // hold no selected key
  const int T0_low = (nqt - 1 - min(4 * kblk + 3, units - 1) / G) * AQ;
  const int kt0 = a.window ? max(0, T0_low - sh.M + 1) / AK : 0;

  const size_t kv_stride = (size_t)sh.H_kv * D;
  const size_t q_stride = (size_t)sh.H_q * D;
  const bf16_t* qb = (const bf16_t*)a.q + (size_t)b * n * q_stride + (size_t)h * D;

  const float scale = a.scale_log2e;
  const int nkt = tmax / AK + 1;

  // The key tiles to walk: from kt0 in window mode; otherwise the tiles in
  // which some row of the block's query tiles selects a key, as the
  // occupancy pass recorded them per group of 32 query rows.  For
  // spread-out selections that is every causal tile; clustered ones (recent
  // keys, sinks) skip the rest.  The block's rows are groups g_lo .. g_hi:
  // two groups for GQA groups of two or more heads, four with one head.
  int count = 0;
  {
    const uint32_t* occ_b = nullptr;
    int g_lo = 0, g_hi = -1;
    if (!a.window && a.occ) {
      const int occ_rows = (n + 31) / 32;
      const int T0_high = (nqt - 1 - (4 * kblk) / G) * AQ;
      g_lo = T0_low / 32;
      g_hi = min((T0_high + AQ - 1) / 32, occ_rows - 1);
      occ_b = a.occ + (size_t)b * occ_rows * a.occ_ld;
    }
    for (int base = 0; base < nkt; base += 256) {
      const int tile = base + tid;
      bool on = tile < nkt && tile >= kt0;
      if (on && occ_b) {
        uint32_t w = 0u;
        for (int gq = g_lo; gq <= g_hi; ++gq) w |= occ_b[(size_t)gq * a.occ_ld + (tile >> 5)];
        on = (w >> (tile & 31)) & 1u;
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
      if (lane == 0) tile_count[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int pos = count;
      for (int w = 0; w < wave; ++w) pos += tile_count[w];
      pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (on) tiles[pos] = (uint16_t)tile;
      count += tile_count[0] + tile_count[1] + tile_count[2] + tile_count[3];
      __syncthreads();
    }
  }

  // K, V and mask rows of the sequence through buffer resources limited to
  // its n rows: loads past them return zeros.  Per-thread byte offsets start
  // at key tile 0 and advance by one tile per prefetch.
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16_t*)a.k_cache + (size_t)b * sh.cap * kv_stride), (short)0, (int)(n * kv_stride * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16_t*)a.v_cache + (size_t)b * sh.cap * kv_stride), (short)0, (int)(n * kv_stride * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t mres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.mask + (size_t)b * n * a.mask_ld), (short)0, (int)(n * a.mask_ld * 4), 0x00020000);
  const uint32_t tile_kv_bytes = (uint32_t)(AK * kv_stride * 2);
  // K and V share the cache layout, so one offset per staged vector serves both
  uint32_t koff[AttnRegs<D>::NK], moff_b[AP];
#pragma unroll
  for (int m = 0; m < AttnRegs<D>::NK; ++m) {
    const int e = tid + 256 * m;
    koff[m] = (uint32_t)(((e / (D / 8)) * kv_stride + (size_t)kvh * D + 8 * (e % (D / 8))) * 2);
  }
  // mask rows of the wave's queries (rows past n read row n - 1; never stored)
#pragma unroll
  for (int i = 0; i < AP; ++i) moff_b[i] = (uint32_t)((size_t)min(T0 + 16 * i + r16, n - 1) * a.mask_ld * 4);

  // next tile's K (and V) and mask words, held in registers while the
  // current tile runs
  AttnRegs<D> rg;
#pragma unroll
  for (int i = 0; i < AP; ++i) rg.mw[i] = make_uint2(0u, 0u);  // not loaded for a sliding window
  auto prefetch = [&](int kt, bool with_v) {
    const uint32_t tk = (uint32_t)kt * tile_kv_bytes;
#pragma unroll
    for (int m = 0; m < AttnRegs<D>::NK; ++m) {
      const uint32_t off = koff[m] + tk;
      rg.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kres, off, 0, 0));
      if (with_v) rg.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vres, off, 0, 0));
    }
    if (!a.window) {
#pragma unroll
      for (int i = 0; i < AP; ++i)
        rg.mw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(mres, moff_b[i] + (uint32_t)kt * 8u, 0, 0));
    }
  };
  // Q^T operands, held for the whole block: lane holds Q[T0 + 16 i + r16][32 s + 8 g .. + 7]
  bf16x8 qreg[AP][D / 32];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    const int t = min(T0 + 16 * i + r16, n - 1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qreg[i][s] = as_bf16x8(ld16(qb + (size_t)t * q_stride + 32 * s + 8 * g));
  }
  // S^T of every query tile i against the staged keys: st[i][c][r] = q . k
  // for the query T0 + 16 i + r16 and the key J0 + 16 c + 4 g + r; sel[i][c]
  // holds the selection bits of those keys (bit r), cut to the causal ones
  // on tiles that reach past the wave's first query
  // (every K operand read from LDS serves all AP query tiles)
  auto scores = [&](int buf, int J0, const uint2 (&mw)[AP], f32x4 (&st)[AP][4], uint32_t (&sel)[AP][4]) {
    // K operands of key block c: key 16 c + r16, dims 32 s + 8 g .. + 7.  The
    // reads of block c + 1 go out before the MFMAs of block c, so the LDS
    // latency hides behind 2 D / 32 MFMAs instead of stalling each pair.
    bf16x8 kf[2][D / 32];
    auto load_k = [&](int c, bf16x8 (&dst)[D / 32]) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) dst[s] = as_bf16x8(lds_read16(&sm.k[buf][16 * c + r16][32 * s + 8 * g]));
    };
    load_k(0, kf[0]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) load_k(c + 1, kf[(c + 1) & 1]);
#pragma unroll
      for (int i = 0; i < AP; ++i) st[i][c] = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int i = 0; i < AP; ++i) st[i][c] = mfma16(kf[c & 1][s], qreg[i][s], st[i][c]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, D / 32, 0);  // LDS reads of block 0
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, D / 32, 0);  // reads of block c + 1
      __builtin_amdgcn_sched_group_barrier(0x008, AP * D / 32, 0);           // MFMAs of block c
    }
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      uint32_t wx = mw[i].x, wy = mw[i].y;
      if (a.window) {  // keys at or past the row's window start (the causal cut follows)
        const int lo = T0 + 16 * i + r16 - sh.M + 1 - J0;
        wx = lo <= 0 ? ~0u : (lo >= 32 ? 0u : ~((1u << lo) - 1u));
        wy = lo <= 32 ? ~0u : (lo >= 64 ? 0u : ~((1u << (lo - 32)) - 1u));
      }
      if (J0 + AK - 1 > T0) {
        const int lim = T0 + 16 * i + r16 - J0;  // last key of the row inside the tile
        wx &= lim >= 31 ? ~0u : (lim < 0 ? 0u : ((2u << lim) - 1u));
        wy &= lim >= 63 ? ~0u : (lim < 32 ? 0u : ((2u << (lim - 32)) - 1u));
      }
      sel[i][0] = wx >> (4 * g);
      sel[i][1] = wx >> (16 + 4 * g);
      sel[i][2] = wy >> (4 * g);
      sel[i][3] = wy >> (16 + 4 * g);
    }
  };
  // all-ones where bit r of w is set, else zero
  auto bitmask = [](uint32_t w, int r) -> uint32_t { return (uint32_t)__builtin_amdgcn_sbfe((int)w, r, 1); };

  // the V operand of the row-sum block: every entry 1.0 (a constant, not an LDS read)
  const bf16x8 ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  // V operand of output block q, contraction step s: keys 32 s + 4 g + 0..3
  // and 32 s + 16 + 4 g + 0..3 (the key order of the P operand) of column
  // 16 q + r16, as two transposing loads; lane r16 of group g points at row
  // 4 g + r16 / 4 (plus 32 s, plus 16), columns 16 q + 4 (r16 % 4) .. + 3
  const int vrow = 4 * g + (r16 >> 2), vcol = 4 * (r16 & 3);
  auto v_operand = [&](int buf, int q, int s) -> bf16x8 {
    const bf16_t* p = &sm.v[buf][32 * s + vrow][16 * q + vcol];
    const v4i16 lo = lds_read_tr4(p);
    const v4i16 hi = lds_read_tr4(p + 16 * (D + 16));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  constexpr int NQ = D / 16 + 1;  // output column blocks, the last one accumulates the row sums
  f32x4 o[AP][NQ];
  float moff[AP];
  // Everything from here to the epilogue is compiled twice: for a block
  // that walks every tile from kt0 (the tile index is the step count, no
  // list lookups) and for one that walks a list.
  auto run = [&](auto dense_c) {
    constexpr bool dense = decltype(dense_c)::value;
    auto kt_of = [&](int i) -> int {
      if constexpr (dense) return kt0 + i;
      else return __builtin_amdgcn_readfirstlane((int)tiles[i]);
    };
    // Walks the listed key tiles: body(kt, buf, mw) computes tile kt from LDS
    // buffer buf with the mask words mw of the wave's rows, while the next
    // listed tile (loaded into registers one tile earlier) is staged into the
    // other buffer; one barrier per tile.
    auto walk = [&](bool with_v, auto&& body) {
      uint2 mw[AP];
      prefetch(kt_of(0), with_v);
      attn_stage<D>(rg, sm, 0, with_v);
  #pragma unroll
      for (int i = 0; i < AP; ++i) mw[i] = rg.mw[i];
      __syncthreads();
      if (1 < count) prefetch(kt_of(1), with_v);
      for (int it = 0; it < count; ++it) {
        body(kt_of(it), it & 1, mw);
        if (it + 1 < count) {
          attn_stage<D>(rg, sm, (it + 1) & 1, with_v);
  #pragma unroll
          for (int i = 0; i < AP; ++i) mw[i] = rg.mw[i];
        }
        __syncthreads();
        if (it + 2 < count) prefetch(kt_of(it + 2), with_v);
      }
    };

    // Every row accumulates O = sum_k p_k v_k and l = sum_k p_k with
    // p_k = exp2(s_k scale - moff) for one fixed offset per row, so the
    // accumulators are never rescaled.  First attempt: the offset is the
    // row's max over the whole first key tile the wave computes (unmasked; any
    // finite offset gives the same softmax in exact arithmetic).  The attempt is kept when l
    // lies in [2^-60, inf) and O is finite for every row of the block, which
    // bounds both underflow of the leading terms and overflow; otherwise the
    // block recomputes with the exact max over the selected keys (a pass over
    // the key tiles without V), for which every p <= 1.
    // O += P V over all key tiles with the offsets in moff; with set_offset the
    // offsets are first taken from the first tile the wave computes
    auto accumulate = [&](bool set_offset) {
  #pragma unroll
      for (int i = 0; i < AP; ++i)
  #pragma unroll
        for (int q = 0; q < NQ; ++q) o[i][q] = zero4();
      bool need_offset = set_offset;  // uniform over the wave
      walk(true, [&](int kt, int buf, const uint2 (&mw)[AP]) {
        const int J0 = kt * AK;
        uint4 pf[AP][2];  // probabilities as bf16, contraction order of the P V step
        f32x4 st[AP][4];
        uint32_t sel[AP][4];
        // MFMA phases at raised wave priority, so that the other wave on the
        // SIMD fills the matrix-core time with its softmax arithmetic
        __builtin_amdgcn_s_setprio(1);
        scores(buf, J0, mw, st, sel);
        __builtin_amdgcn_s_setprio(0);
        // V operands of output blocks 0 and 1, read while the softmax runs;
        // each later block's operands are read two blocks ahead of its MFMAs
        bf16x8 vf[3][2];
  #pragma unroll
        for (int q = 0; q < 2; ++q)
  #pragma unroll
          for (int s = 0; s < 2; ++s) vf[q][s] = v_operand(buf, q, s);
  #pragma unroll
        for (int i = 0; i < AP; ++i) {
          if (need_offset) {  // the row's offset: max over the first computed tile
            float m = -INFINITY;
  #pragma unroll
            for (int c = 0; c < 4; ++c) m = fmaxf(m, fmaxf(fmaxf(st[i][c][0], st[i][c][1]), fmaxf(st[i][c][2], st[i][c][3])));
            m = fmaxf(m, __shfl_xor(m, 16, WAVE));
            m = fmaxf(m, __shfl_xor(m, 32, WAVE));
            moff[i] = m * scale;
          }
          // exponent s scale - offset, replaced by -inf (exp2 -> 0) where the
          // key is not selected
          uint32_t pk[4][2];
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            float x[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t m = bitmask(sel[i][c], r);
              x[r] = __uint_as_float((__float_as_uint(fmaf(st[i][c][r], scale, -moff[i])) & m) | (0xff800000u & ~m));
            }
  #pragma unroll
            for (int r = 0; r < 4; r += 2)
              pk[c][r / 2] = cvt_pk_bf16(__builtin_amdgcn_exp2f(x[r]), __builtin_amdgcn_exp2f(x[r + 1]));
          }
          // contraction step s covers key blocks 2 s and 2 s + 1
  #pragma unroll
          for (int s = 0; s < 2; ++s) pf[i][s] = make_uint4(pk[2 * s][0], pk[2 * s][1], pk[2 * s + 1][0], pk[2 * s + 1][1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        need_offset = false;
        __builtin_amdgcn_s_setprio(1);
        // O += P V over the output blocks, then the ones block
  #pragma unroll
        for (int q = 0; q < NQ - 1; ++q) {
          if (q + 2 < NQ - 1)
  #pragma unroll
            for (int s = 0; s < 2; ++s) vf[(q + 2) % 3][s] = v_operand(buf, q + 2, s);
  #pragma unroll
          for (int s = 0; s < 2; ++s)
  #pragma unroll
            for (int i = 0; i < AP; ++i) o[i][q] = mfma16(as_bf16x8(pf[i][s]), vf[q % 3][s], o[i][q]);
        }
  #pragma unroll
        for (int s = 0; s < 2; ++s)
  #pragma unroll
          for (int i = 0; i < AP; ++i) o[i][NQ - 1] = mfma16(as_bf16x8(pf[i][s]), ones, o[i][NQ - 1]);
  #pragma unroll
        for (int q = 0; q < NQ - 1; ++q) {
          if (q + 2 < NQ - 1) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);  // reads of block q + 2
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * AP, 1);                // MFMAs of block q
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * AP, 1);  // the ones block
        __builtin_amdgcn_s_setprio(0);
      });
    };

    accumulate(true);
    // keep the result unless some row of the block is out of range
    bool bad = false;
  #pragma unroll
    for (int i = 0; i < AP; ++i)
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l = o[i][NQ - 1][r];
        bad |= !(l >= 0x1p-60f && l < INFINITY);
  #pragma unroll
        for (int q = 0; q < NQ - 1; ++q) bad |= !(fabsf(o[i][q][r]) < INFINITY);
      }
    if (__syncthreads_or(bad)) {
      // exact maxima over the selected keys (a pass without V), then again
      float mx[AP];
  #pragma unroll
      for (int i = 0; i < AP; ++i) mx[i] = -INFINITY;
      walk(false, [&](int kt, int buf, const uint2 (&mw)[AP]) {
        f32x4 st[AP][4];
        uint32_t sel[AP][4];
        scores(buf, kt * AK, mw, st, sel);
  #pragma unroll
        for (int i = 0; i < AP; ++i) {
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            float v[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) {  // the score where selected, -inf elsewhere
              const uint32_t m = bitmask(sel[i][c], r);
              v[r] = __uint_as_float((__float_as_uint(st[i][c][r]) & m) | (0xff800000u & ~m));
            }
            mx[i] = fmaxf(mx[i], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      });
  #pragma unroll
      for (int i = 0; i < AP; ++i) {
        float m = fmaxf(mx[i], __shfl_xor(mx[i], 16, WAVE));
        m = fmaxf(m, __shfl_xor(m, 32, WAVE));
        moff[i] = m == -INFINITY ? 0.f : m * scale;
      }
      __syncthreads();
      accumulate(false);
    }
  };
  if (count == nkt - kt0) run(std::true_type{});
  else run(std::false_type{});
  if (!active) return;

  // epilogue: out = g O_s + (1 - g) O_L for rows t = T0 + 16 i + 4 g + r;
  // the row sum of a row is in its ones block
  const float* gate = a.gate_part;
  const float* olin = a.o_lin;
  bf16_t* out = (bf16_t*)a.out;
#pragma unroll
  for (int i = 0; i < AP; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = T0 + 16 * i + 4 * g + r;
      if (t >= n) continue;
      const float ir = 1.f / o[i][NQ - 1][r];  // every causal row selects at least itself
      const size_t row = (size_t)b * n + t;
      const float gv = sigmoidf(gate[row * sh.H_q + h]);
      const float* ol = olin + (row * sh.H_q + h) * D;
      bf16_t* op = out + (row * sh.H_q + h) * D;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const int dv = 16 * q + r16;
        op[dv] = (bf16_t)f2bf(gv * o[i][q][r] * ir + (1.f - gv) * ol[dv]);
      }
    }
  }
}

bool attn_mfma_supported(const Shape& sh) {
  return sh.dtype == 1 && (sh.d == 64 || sh.d == 128);
}

int64_t attn_mask_ld(int n) { return (int64_t)((((n + 31) / 32) + 1) / 2 * 2); }

hipError_t launch_attn_prefill_mfma(const AttnMaskArgs& a, hipStream_t st) {
  // buffer resources address a sequence's K, V and mask rows with 31-bit offsets
  if ((size_t)a.n * a.sh.H_kv * a.sh.d * 2 > 0x7fffffffu || (size_t)a.n * a.mask_ld * 4 > 0x7fffffffu)
    return hipErrorInvalidValue;
  const int G = a.sh.H_q / a.sh.H_kv;
  const int units = (a.n + AQ - 1) / AQ * G;
  const dim3 grid((unsigned)((units + 3) / 4 * a.sh.B * a.sh.H_kv));
  if (a.sh.d == 128) klaunch(k_attn_prefill_mfma<128>, grid, dim3(256), 0, st, a);
  else klaunch(k_attn_prefill_mfma<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
