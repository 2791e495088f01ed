// Linear-attention branch of the LISA prefill on bf16 MFMA ("LISA", arXiv
// 2607.19358v1, Section 3.3 Eqs. 3-4: S_t = S_{t-1} + phi(k_t)^T v_t,
// o_t = phi(q_t) S_t / (phi(q_t) . z_t) with z_t = z_{t-1} + phi(k_t) and
// phi = elu + 1), computed in chunks of 64 tokens:
//
//   A   = (phi(Q_c) phi(K_c)^T) masked to key <= query (diagonal included)
//   num = A V_c + phi(Q_c) S          den = rowsum(A) + phi(Q_c) . z
//   S  += phi(K_c)^T V_c              z  += column sums of phi(K_c)
//
// where S and z are the state before the chunk.  A sequence is cut into
// segments of whole chunks so that many blocks work at once:
//   k_lin_seg_sums   the state increment of every segment (or, in place,
//                    of the whole sequence);
//   k_lin_seg_prefix the state entering every segment and the final state;
//   k_lin_chunks     one block per segment walks its chunks and writes the
//                    outputs.
//
// Precision: the state is an fp32 MFMA accumulator.  phi(K) enters the
// state update as a bf16 pair hi + lo (hi = bf16(phi(k)), lo = bf16(phi(k) -
// hi)), and S enters phi(Q) S as such a pair too, so both products carry the
// fp32 values to about 2^-17; V is bf16 already.  phi(Q), phi(K) in A and A
// itself are rounded to bf16 once.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"
#include "lisa_prefill.h"

namespace lisa {

constexpr int LC = 64;          // chunk length
constexpr int LPAD = 8;         // LDS row padding (elements)

// One wave per 16 value columns of the state: D / 16 waves.
template <int D>
struct LinCfg {
  static constexpr int W = D / 16;        // waves per block
  static constexpr int T = 64 * W;        // threads per block
  static constexpr int WPI = W / 4;       // waves per 16-row query block of a chunk
};

template <int D>
struct LinShared {
  bf16_t q[LC][D + LPAD];       // phi(Q) rows, bf16
  bf16_t k[LC][D + LPAD];       // phi(K) rows, bf16 (hi)
  bf16_t kt_hi[D][LC + LPAD];   // phi(K) transposed, hi part
  bf16_t kt_lo[D][LC + LPAD];   // phi(K) transposed, lo part
  bf16_t vt[D][LC + LPAD];      // V transposed
  bf16_t a[LC][LC + LPAD];      // masked intra-chunk scores
  float z[2][D];                // normaliser before / after the chunk
  float rs[LinCfg<D>::WPI + 1][LC];  // partial row sums of A; last: phi(q) . z
};

template <int D>
struct LinSumShared {
  bf16_t kt_hi[D][LC + LPAD];
  bf16_t kt_lo[D][LC + LPAD];
  bf16_t vt[D][LC + LPAD];
};

// Global -> register prefetch of one chunk.  A thread holds, per matrix,
// NP pairs of 16-byte vectors: tokens 2 tau and 2 tau + 1 (tau = lane % 32)
// at columns 8 c8, c8 = 2 (wave + W m) + lane / 32.  Holding two adjacent
// tokens lets the transposed LDS copies be written as packed token pairs:
// 32 consecutive dwords of one row per half wave, free of bank conflicts.
template <int D, bool WITH_Q>
struct ChunkRegs {
  static constexpr int NP = LC * D / 16 / LinCfg<D>::T;
  uint4 q[WITH_Q ? 2 * NP : 1], k[2 * NP], v[2 * NP];
};

template <int D>
__device__ __forceinline__ void pair_coords(int m, int& tau, int& c8) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  tau = lane & 31;
  c8 = 2 * (wave + LinCfg<D>::W * m) + (lane >> 5);
}

template <int D, bool WITH_Q>
__device__ __forceinline__ void chunk_load(ChunkRegs<D, WITH_Q>& r, const bf16_t* qb, const bf16_t* kb,
                                           const bf16_t* vb, size_t tok_stride, int t0, int n) {
#pragma unroll
  for (int m = 0; m < ChunkRegs<D, WITH_Q>::NP; ++m) {
    int tau, c8;
    pair_coords<D>(m, tau, c8);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // clamped: every load is issued unconditionally
      const size_t off = (size_t)min(t0 + 2 * tau + u, n - 1) * tok_stride + 8 * c8;
      if constexpr (WITH_Q) r.q[2 * m + u] = ld16(qb + off);
      r.k[2 * m + u] = ld16(kb + off);
      r.v[2 * m + u] = ld16(vb + off);
    }
  }
}

// Registers -> LDS: phi applied, hi/lo split, transposed copies.  Tokens at
// or past n are written as zeros (phi(0) = 1 would otherwise count them).
template <int D, bool WITH_Q, typename SM>
__device__ __forceinline__ void chunk_store(const ChunkRegs<D, WITH_Q>& r, SM& sm, int t0, int n) {
#pragma unroll
  for (int m = 0; m < ChunkRegs<D, WITH_Q>::NP; ++m) {
    int tau, c8;
    pair_coords<D>(m, tau, c8);
    const bool v0 = t0 + 2 * tau < n, v1 = t0 + 2 * tau + 1 < n;
    float k0[8], k1[8];
    Vec<bf16_t>::unpack(r.k[2 * m], k0);
    Vec<bf16_t>::unpack(r.k[2 * m + 1], k1);
    // element e of both tokens as one packed pair: the transposed row's dword
    uint32_t kh[8], kl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_pk(v0 ? phi(k0[e]) : 0.f, v1 ? phi(k1[e]) : 0.f, kh[e], kl[e]);
    const uint4 va = v0 ? r.v[2 * m] : make_uint4(0u, 0u, 0u, 0u);
    const uint4 vb = v1 ? r.v[2 * m + 1] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t a4[4] = {va.x, va.y, va.z, va.w}, b4[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * c8 + e;
      *reinterpret_cast<uint32_t*>(&sm.kt_hi[row][2 * tau]) = kh[e];
      *reinterpret_cast<uint32_t*>(&sm.kt_lo[row][2 * tau]) = kl[e];
      const uint32_t x = a4[e / 2], y = b4[e / 2];
      *reinterpret_cast<uint32_t*>(&sm.vt[row][2 * tau]) =
          (e & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
    }
    if constexpr (WITH_Q) {
      // row-major phi(K) (hi) of each token: regroup the pairs by token
      uint4 r0, r1;
      uint32_t* p0 = &r0.x;
      uint32_t* p1 = &r1.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p0[j] = __builtin_amdgcn_perm(kh[2 * j + 1], kh[2 * j], 0x05040100u);
        p1[j] = __builtin_amdgcn_perm(kh[2 * j + 1], kh[2 * j], 0x07060302u);
      }
      *reinterpret_cast<uint4*>(&sm.k[2 * tau][8 * c8]) = r0;
      *reinterpret_cast<uint4*>(&sm.k[2 * tau + 1][8 * c8]) = r1;
      float q0[8], q1[8];
      Vec<bf16_t>::unpack(r.q[2 * m], q0);
      Vec<bf16_t>::unpack(r.q[2 * m + 1], q1);
      uint4 s0, s1;
      uint32_t* w0 = &s0.x;
      uint32_t* w1 = &s1.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0[j] = cvt_pk_bf16(v0 ? phi(q0[2 * j]) : 0.f, v0 ? phi(q0[2 * j + 1]) : 0.f);
        w1[j] = cvt_pk_bf16(v1 ? phi(q1[2 * j]) : 0.f, v1 ? phi(q1[2 * j + 1]) : 0.f);
      }
      *reinterpret_cast<uint4*>(&sm.q[2 * tau][8 * c8]) = s0;
      *reinterpret_cast<uint4*>(&sm.q[2 * tau + 1][8 * c8]) = s1;
    }
  }
}

// S[dk][dv] += sum_tok phi(K)[tok][dk] V[tok][dv] over the staged chunk, for
// the wave's 16 dv columns: tiles p over dk blocks of 16.
template <int D, typename SM>
__device__ __forceinline__ void state_update(f32x4 (&S)[D / 16], const SM& sm, int wave) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < LC / 32; ++s) {
    const bf16x8 bv = as_bf16x8(lds_read16(&sm.vt[16 * wave + r16][32 * s + 8 * g]));
#pragma unroll
    for (int p = 0; p < D / 16; ++p) {
      const bf16x8 ah = as_bf16x8(lds_read16(&sm.kt_hi[16 * p + r16][32 * s + 8 * g]));
      const bf16x8 al = as_bf16x8(lds_read16(&sm.kt_lo[16 * p + r16][32 * s + 8 * g]));
      S[p] = mfma16(ah, bv, S[p]);
      S[p] = mfma16(al, bv, S[p]);
    }
  }
}

// Column sums of phi(K) over the staged chunk, shared by every wave: wave w
// sums dk rows 16 w .. 16 w + 15, lane l row 16 w + l % 16 over the 16 tokens
// of quarter l / 16; the quarters are then added across lanes.  Lanes 0..15
// return the sum of row ksum_row(wave, lane) (other lanes: partial values).
__device__ __forceinline__ int ksum_row(int wave, int lane) { return 16 * wave + (lane & 15); }

template <int D, typename SM>
__device__ __forceinline__ float chunk_ksum(const SM& sm, int wave, int lane) {
  static_assert(D / LinCfg<D>::W == 16, "16 rows per wave");
  const int dk = ksum_row(wave, lane), c0 = 16 * (lane >> 4);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 16; c += 8) {
    float h[8], l[8];
    Vec<bf16_t>::load(&sm.kt_hi[dk][c0 + c], h);
    Vec<bf16_t>::load(&sm.kt_lo[dk][c0 + c], l);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += h[u] + l[u];
  }
  acc += __shfl_xor(acc, 16, WAVE);
  acc += __shfl_xor(acc, 32, WAVE);
  return acc;
}

// Lane's element (row 4g + r, column lane % 16) of an MFMA tile -> position
// of the wave's state tile in the [D][D] array.
__device__ __forceinline__ size_t tile_off(int D, int p, int qg, int lane, int r) {
  return (size_t)(16 * p + 4 * (lane >> 4) + r) * D + 16 * qg + (lane & 15);
}

// ---------------------------------------------------------------------------
// state increments: block (b, h, segment); wave w owns dv columns
// [16 w, 16 w + 16).  Segment mode writes the increment to `seg`; in-place
// mode (one segment) adds it to S and z.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(LinCfg<D>::T) void k_lin_seg_sums(LinearChunkArgs a) {
  __shared__ LinSumShared<D> sm;
  const Shape& sh = a.sh;
  const int seg = blockIdx.x % a.nseg;
  const int bh = blockIdx.x / a.nseg;
  const int h = bh % sh.H_L, b = bh / sh.H_L;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const size_t tok_stride = (size_t)sh.H_L * D;
  const bf16_t* kb = (const bf16_t*)a.k_lin + (size_t)b * a.n * tok_stride + (size_t)h * D;
  const bf16_t* vb = (const bf16_t*)a.v_lin + (size_t)b * a.n * tok_stride + (size_t)h * D;
  const int t_begin = seg * a.seg_len;
  const int t_end = min(a.n, t_begin + a.seg_len);

  f32x4 S[D / 16];
  float* Sg = a.S + (size_t)bh * D * D;
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[p][r] = a.in_place ? Sg[tile_off(D, p, wave, lane, r)] : 0.f;
  const int zrow = ksum_row(wave, lane);  // lanes 0..15 keep z of this row
  float zacc = (a.in_place && lane < 16) ? a.z[(size_t)bh * D + zrow] : 0.f;

  ChunkRegs<D, false> cr;
  if (t_begin < t_end) chunk_load<D, false>(cr, nullptr, kb, vb, tok_stride, t_begin, a.n);
  for (int t0 = t_begin; t0 < t_end; t0 += LC) {
    __syncthreads();  // previous chunk's readers are done
    chunk_store<D, false>(cr, sm, t0, t_end);
    __syncthreads();
    if (t0 + LC < t_end) chunk_load<D, false>(cr, nullptr, kb, vb, tok_stride, t0 + LC, a.n);
    state_update<D>(S, sm, wave);
    zacc += chunk_ksum<D>(sm, wave, lane);
  }
  float* dst = a.in_place ? Sg : a.seg_state + ((size_t)bh * a.nseg + seg) * (D * D + D);
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[tile_off(D, p, wave, lane, r)] = S[p][r];
  if (lane < 16) {
    if (a.in_place) a.z[(size_t)bh * D + zrow] = zacc;
    else dst[D * D + zrow] = zacc;
  }
}

// ---------------------------------------------------------------------------
// exclusive scan over segments: seg_state[s] <- state entering segment s;
// S, z <- the state after the last segment.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lin_seg_prefix(LinearChunkArgs a) {
  const int D = a.sh.d;
  const int per = D * D + D;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= per) return;
  float* Sg = a.S + (size_t)bh * D * D;
  float* zg = a.z + (size_t)bh * D;
  float run = e < D * D ? Sg[e] : zg[e - D * D];
  float* seg = a.seg_state + (size_t)bh * a.nseg * per + e;
  for (int s = 0; s < a.nseg; ++s) {
    const float inc = seg[(size_t)s * per];
    seg[(size_t)s * per] = run;
    run += inc;
  }
  if (e < D * D) Sg[e] = run;
  else zg[e - D * D] = run;
}

// ---------------------------------------------------------------------------
// chunked outputs: block (b, h, segment), starting from the segment's state.
// Wave w owns dv columns [16 w, 16 w + 16) of S and of the outputs; the
// intra-chunk score tiles are shared out WPI waves per query block.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(LinCfg<D>::T) void k_lin_chunks(LinearChunkArgs a) {
  __shared__ LinShared<D> sm;
  constexpr int WPI = LinCfg<D>::WPI;
  const Shape& sh = a.sh;
  const bool normalized = !(sh.flags & 1u);
  const int seg = blockIdx.x % a.nseg;
  const int bh = blockIdx.x / a.nseg;
  const int h = bh % sh.H_L, b = bh / sh.H_L;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t tok_stride = (size_t)sh.H_L * D;
  const size_t base = (size_t)b * a.n * tok_stride + (size_t)h * D;
  const bf16_t* qb = (const bf16_t*)a.q_lin + base;
  const bf16_t* kb = (const bf16_t*)a.k_lin + base;
  const bf16_t* vb = (const bf16_t*)a.v_lin + base;
  const int t_begin = seg * a.seg_len;
  const int t_end = min(a.n, t_begin + a.seg_len);
  if (t_begin >= t_end) return;

  const float* st = a.seg_state + ((size_t)bh * a.nseg + seg) * (D * D + D);
  f32x4 S[D / 16];
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[p][r] = st[tile_off(D, p, wave, lane, r)];
  if (tid < D) sm.z[0][tid] = st[D * D + tid];
  int zc = 0;

  ChunkRegs<D, true> cr;
  chunk_load<D, true>(cr, qb, kb, vb, tok_stride, t_begin, a.n);
  for (int t0 = t_begin; t0 < t_end; t0 += LC) {
    __syncthreads();  // readers of the previous chunk are done
    chunk_store<D, true>(cr, sm, t0, t_end);
    __syncthreads();
    if (t0 + LC < t_end) chunk_load<D, true>(cr, qb, kb, vb, tok_stride, t0 + LC, a.n);

    // intra-chunk scores of query block ib, key blocks kbk = sub, sub + WPI,
    // ... up to ib (plus the zero block above the diagonal that the A V
    // product reads when ib is even)
    const int ib = wave / WPI, sub = wave % WPI;
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4 / WPI; ++kk) {
      const int kbk = sub + WPI * kk;
      if (kbk > (ib | 1)) break;
      f32x4 acc = zero4();
      if (kbk <= ib) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 qa = as_bf16x8(lds_read16(&sm.q[16 * ib + r16][32 * s + 8 * g]));
          const bf16x8 kk8 = as_bf16x8(lds_read16(&sm.k[16 * kbk + r16][32 * s + 8 * g]));
          acc = mfma16(qa, kk8, acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * g + r, j = 16 * kbk + r16;
        const uint32_t ab = j <= i ? (cvt_pk_bf16(acc[r], 0.f) & 0xffffu) : 0u;
        sm.a[i][j] = (bf16_t)ab;
        rsum[r] += bf2f(ab);
      }
    }
    // partial row sums: rows 16 ib + 4 g + r, summed over the 16 key lanes
#pragma unroll
    for (int r = 0; r < 4; ++r) rsum[r] = group_sum(rsum[r], 16);
    if (r16 < 4)
      sm.rs[sub][16 * ib + 4 * g + r16] = r16 == 0 ? rsum[0] : r16 == 1 ? rsum[1] : r16 == 2 ? rsum[2] : rsum[3];
    {
      // phi(q) . z, every wave for LC / W rows: lane l takes 16 dims of row
      // LC / W * wave + l / SL, the SL lanes of a row are then summed
      constexpr int RPW = LC / LinCfg<D>::W, SL = WAVE / RPW;
      static_assert(D / SL == 16, "16 dims per lane");
      const int i = RPW * wave + lane / SL, c0 = 16 * (lane % SL);
      float qz = 0.f;
#pragma unroll
      for (int c = 0; c < 16; c += 8) {
        float qf[8];
        Vec<bf16_t>::load(&sm.q[i][c0 + c], qf);
#pragma unroll
        for (int u = 0; u < 8; ++u) qz = fmaf(qf[u], sm.z[zc][c0 + c + u], qz);
      }
#pragma unroll
      for (int o = 1; o < SL; o <<= 1) qz += __shfl_xor(qz, o, WAVE);
      if (lane % SL == 0) sm.rs[WPI][i] = qz;
    }
    __syncthreads();  // A and the row sums complete

    // num^T = V^T A^T + S^T phi(Q)^T for every query block, the wave's dv
    // block: the operands of num = A V + phi(Q) S in swapped MFMA order, so
    // that a lane ends up with four consecutive dv columns of one query row
    // (one float4 store).  S enters straight from the accumulator: lane
    // (r16, g) holds dk rows 32 pp + 4 g + r and 32 pp + 16 + 4 g + r of
    // column r16, so phi(Q) is read in that same contraction order.
    uint4 shi[D / 32], slo[D / 32];
#pragma unroll
    for (int pp = 0; pp < D / 32; ++pp) {
      uint32_t h4[4], l4[4];
      split_pk(S[2 * pp][0], S[2 * pp][1], h4[0], l4[0]);
      split_pk(S[2 * pp][2], S[2 * pp][3], h4[1], l4[1]);
      split_pk(S[2 * pp + 1][0], S[2 * pp + 1][1], h4[2], l4[2]);
      split_pk(S[2 * pp + 1][2], S[2 * pp + 1][3], h4[3], l4[3]);
      shi[pp] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
      slo[pp] = make_uint4(l4[0], l4[1], l4[2], l4[3]);
    }
#pragma unroll
    for (int ibq = 0; ibq < 4; ++ibq) {
      f32x4 num = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && ibq < 2) break;
        const bf16x8 aa = as_bf16x8(lds_read16(&sm.a[16 * ibq + r16][32 * s + 8 * g]));
        const bf16x8 vv = as_bf16x8(lds_read16(&sm.vt[16 * wave + r16][32 * s + 8 * g]));
        num = mfma16(vv, aa, num);  // [dv][query]
      }
#pragma unroll
      for (int pp = 0; pp < D / 32; ++pp) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(&sm.q[16 * ibq + r16][32 * pp + 4 * g]);
        const uint2 x1 = *reinterpret_cast<const uint2*>(&sm.q[16 * ibq + r16][32 * pp + 16 + 4 * g]);
        const bf16x8 qa = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
        num = mfma16(as_bf16x8(shi[pp]), qa, num);
        num = mfma16(as_bf16x8(slo[pp]), qa, num);
      }
      // lane holds row i = 16 ibq + r16, dv columns 16 wave + 4 g .. + 3
      const int i = 16 * ibq + r16;
      const int t = t0 + i;
      float den = sm.rs[WPI][i];
#pragma unroll
      for (int u = 0; u < WPI; ++u) den += sm.rs[u][i];
      if (t < t_end) {
        const float inv = normalized ? __builtin_amdgcn_rcpf(den) : 1.f;
        *reinterpret_cast<float4*>(a.o_lin + ((size_t)b * a.n + t) * tok_stride + (size_t)h * D + 16 * wave + 4 * g) =
            make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
      }
    }
    // state and normaliser after the chunk
    state_update<D>(S, sm, wave);
    {
      const float ks = chunk_ksum<D>(sm, wave, lane);
      const int dk = ksum_row(wave, lane);
      if (lane < 16) sm.z[zc ^ 1][dk] = sm.z[zc][dk] + ks;
    }
    zc ^= 1;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool linear_mfma_supported(const Shape& sh) { return sh.dtype == 1 && (sh.d == 64 || sh.d == 128); }

// Compute units of the current device (256 where it cannot be queried).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cached[dev] = c;
  }
  return cached[dev];
}

// Segments per (sequence, head): the chunk kernel holds one block per CU (its
// LDS), so the blocks are sized to come out at no more than one per CU.
void linear_segments(const Shape& sh, int n, int& nseg, int& seg_len) {
  const int chunks = (n + LC - 1) / LC;
  const int bh = sh.B * sh.H_L;
  int want = max(1, device_cu_count() / bh);
  want = max(1, min(want, chunks));
  const int cps = (chunks + want - 1) / want;
  seg_len = cps * LC;
  nseg = (n + seg_len - 1) / seg_len;
}

size_t linear_seg_floats(const Shape& sh, int n) {
  int nseg, seg_len;
  linear_segments(sh, n, nseg, seg_len);
  return (size_t)sh.B * sh.H_L * nseg * (sh.d * sh.d + sh.d);
}

hipError_t launch_linear_seg_sums(const LinearChunkArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.sh.B * a.sh.H_L * a.nseg));
  if (a.sh.d == 128) klaunch(k_lin_seg_sums<128>, grid, dim3(LinCfg<128>::T), 0, st, a);
  else klaunch(k_lin_seg_sums<64>, grid, dim3(LinCfg<64>::T), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_linear_seg_prefix(const LinearChunkArgs& a, hipStream_t st) {
  const int per = a.sh.d * a.sh.d + a.sh.d;
  const dim3 grid((unsigned)((per + 255) / 256), (unsigned)(a.sh.B * a.sh.H_L));
  klaunch(k_lin_seg_prefix, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_linear_chunks(const LinearChunkArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.sh.B * a.sh.H_L * a.nseg));
  if (a.sh.d == 128) klaunch(k_lin_chunks<128>, grid, dim3(LinCfg<128>::T), 0, st, a);
  else klaunch(k_lin_chunks<64>, grid, dim3(LinCfg<64>::T), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
