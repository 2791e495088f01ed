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
constexpr int LT = 256;         // threads per block (4 waves)
constexpr int LPAD = 8;         // LDS row padding (elements)

template <int D>
struct LinShared {
  bf16_t q[LC][D + LPAD];       // phi(Q) rows, bf16
  bf16_t k[LC][D + LPAD];       // phi(K) rows, bf16 (hi)
  bf16_t kt_hi[D][LC + LPAD];   // phi(K) transposed, hi part
  bf16_t kt_lo[D][LC + LPAD];   // phi(K) transposed, lo part
  bf16_t vt[D][LC + LPAD];      // V transposed
  bf16_t a[LC][LC + LPAD];      // masked intra-chunk scores
  float z[2][D];                // normaliser before / after the chunk
  float den[LC];
};

template <int D>
struct LinSumShared {
  bf16_t kt_hi[D][LC + LPAD];
  bf16_t kt_lo[D][LC + LPAD];
  bf16_t vt[D][LC + LPAD];
};

// Global -> register prefetch of one chunk.  A thread holds, per matrix,
// NP pairs of 16-byte vectors: tokens 2 tau and 2 tau + 1 (tau = lane % 32)
// at columns 8 c8, c8 = 2 (wave + 4 m) + lane / 32.  Holding two adjacent
// tokens lets the transposed LDS copies be written as packed token pairs:
// 32 consecutive dwords of one row per half wave, free of bank conflicts.
template <int D, bool WITH_Q>
struct ChunkRegs {
  static constexpr int NP = LC * D / 16 / LT;
  uint4 q[WITH_Q ? 2 * NP : 1], k[2 * NP], v[2 * NP];
};

__device__ __forceinline__ void pair_coords(int m, int& tau, int& c8) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  tau = lane & 31;
  c8 = 2 * (wave + 4 * m) + (lane >> 5);
}

template <int D, bool WITH_Q>
__device__ __forceinline__ void chunk_load(ChunkRegs<D, WITH_Q>& r, const bf16_t* qb, const bf16_t* kb,
                                           const bf16_t* vb, size_t tok_stride, int t0, int n) {
#pragma unroll
  for (int m = 0; m < ChunkRegs<D, WITH_Q>::NP; ++m) {
    int tau, c8;
    pair_coords(m, tau, c8);
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

__device__ __forceinline__ void split_hi_lo(float f, uint32_t& hi, uint32_t& lo) {
  hi = f2bf(f);
  lo = f2bf(f - bf2f(hi));
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&h)[8]) {
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// Registers -> LDS: phi applied, hi/lo split, transposed copies.  Tokens at
// or past n are written as zeros (phi(0) = 1 would otherwise count them).
template <int D, bool WITH_Q, typename SM>
__device__ __forceinline__ void chunk_store(const ChunkRegs<D, WITH_Q>& r, SM& sm, int t0, int n) {
#pragma unroll
  for (int m = 0; m < ChunkRegs<D, WITH_Q>::NP; ++m) {
    int tau, c8;
    pair_coords(m, tau, c8);
    uint32_t kh[2][8], kl[2][8], vv[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = 2 * tau + u;
      const bool valid = t0 + tok < n;
      float kf[8];
      Vec<bf16_t>::unpack(r.k[2 * m + u], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) split_hi_lo(valid ? phi(kf[e]) : 0.f, kh[u][e], kl[u][e]);
      const uint4 v = valid ? r.v[2 * m + u] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[u][2 * e] = vw[e] & 0xffffu;
        vv[u][2 * e + 1] = vw[e] >> 16;
      }
      if constexpr (WITH_Q) {
        *reinterpret_cast<uint4*>(&sm.k[tok][8 * c8]) = pack8(kh[u]);
        float qf[8];
        Vec<bf16_t>::unpack(r.q[2 * m + u], qf);
        uint32_t qh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qh[e] = f2bf(valid ? phi(qf[e]) : 0.f);
        *reinterpret_cast<uint4*>(&sm.q[tok][8 * c8]) = pack8(qh);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * c8 + e;
      *reinterpret_cast<uint32_t*>(&sm.kt_hi[row][2 * tau]) = kh[0][e] | (kh[1][e] << 16);
      *reinterpret_cast<uint32_t*>(&sm.kt_lo[row][2 * tau]) = kl[0][e] | (kl[1][e] << 16);
      *reinterpret_cast<uint32_t*>(&sm.vt[row][2 * tau]) = vv[0][e] | (vv[1][e] << 16);
    }
  }
}

// S[dk][dv] += sum_tok phi(K)[tok][dk] V[tok][dv] over the staged chunk, for
// the wave's dv blocks: tiles (p, q) with p over dk blocks of 16.
template <int D, typename SM>
__device__ __forceinline__ void state_update(f32x4 (&S)[D / 16][D / 64], const SM& sm, int wave) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < LC / 32; ++s) {
    bf16x8 bv[D / 64];
#pragma unroll
    for (int q = 0; q < D / 64; ++q)
      bv[q] = as_bf16x8(lds_read16(&sm.vt[16 * (wave * (D / 64) + q) + r16][32 * s + 8 * g]));
#pragma unroll
    for (int p = 0; p < D / 16; ++p) {
      const bf16x8 ah = as_bf16x8(lds_read16(&sm.kt_hi[16 * p + r16][32 * s + 8 * g]));
      const bf16x8 al = as_bf16x8(lds_read16(&sm.kt_lo[16 * p + r16][32 * s + 8 * g]));
#pragma unroll
      for (int q = 0; q < D / 64; ++q) {
        S[p][q] = mfma16(ah, bv[q], S[p][q]);
        S[p][q] = mfma16(al, bv[q], S[p][q]);
      }
    }
  }
}

// Column sum of phi(K) over the staged chunk for dk = threadIdx.x (< D).
template <int D, typename SM>
__device__ __forceinline__ float chunk_ksum(const SM& sm, int dk) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < LC; c += 8) {
    float h[8], l[8];
    Vec<bf16_t>::load(&sm.kt_hi[dk][c], h);
    Vec<bf16_t>::load(&sm.kt_lo[dk][c], l);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += h[u] + l[u];
  }
  return acc;
}

// Lane's element (row 4g + r, column lane % 16) of an MFMA tile -> position
// of the wave's state tile in the [D][D] array.
__device__ __forceinline__ size_t tile_off(int D, int p, int qg, int lane, int r) {
  return (size_t)(16 * p + 4 * (lane >> 4) + r) * D + 16 * qg + (lane & 15);
}

// ---------------------------------------------------------------------------
// state increments: block (b, h, segment); wave w owns dv columns
// [D/4 w, D/4 (w+1)).  Segment mode writes the increment to `seg`; in-place
// mode (one segment) adds it to S and z.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(LT) void k_lin_seg_sums(LinearChunkArgs a) {
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

  f32x4 S[D / 16][D / 64];
  float* Sg = a.S + (size_t)bh * D * D;
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int q = 0; q < D / 64; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[p][q][r] = a.in_place ? Sg[tile_off(D, p, wave * (D / 64) + q, lane, r)] : 0.f;
  float zacc = (a.in_place && tid < D) ? a.z[(size_t)bh * D + tid] : 0.f;

  ChunkRegs<D, false> cr;
  if (t_begin < t_end) chunk_load<D, false>(cr, nullptr, kb, vb, tok_stride, t_begin, a.n);
  for (int t0 = t_begin; t0 < t_end; t0 += LC) {
    __syncthreads();  // previous chunk's readers are done
    chunk_store<D, false>(cr, sm, t0, t_end);
    __syncthreads();
    if (t0 + LC < t_end) chunk_load<D, false>(cr, nullptr, kb, vb, tok_stride, t0 + LC, a.n);
    state_update<D>(S, sm, wave);
    if (tid < D) zacc += chunk_ksum<D>(sm, tid);
  }
  float* dst = a.in_place ? Sg : a.seg_state + ((size_t)bh * a.nseg + seg) * (D * D + D);
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int q = 0; q < D / 64; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[tile_off(D, p, wave * (D / 64) + q, lane, r)] = S[p][q][r];
  if (tid < D) {
    if (a.in_place) a.z[(size_t)bh * D + tid] = zacc;
    else dst[D * D + tid] = zacc;
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
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(LT) void k_lin_chunks(LinearChunkArgs a) {
  __shared__ LinShared<D> sm;
  constexpr int NQ = D / 64;  // dv blocks of 16 per wave
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
  f32x4 S[D / 16][NQ];
#pragma unroll
  for (int p = 0; p < D / 16; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[p][q][r] = st[tile_off(D, p, wave * NQ + q, lane, r)];
  if (tid < D) sm.z[0][tid] = st[D * D + tid];
  int zc = 0;

  ChunkRegs<D, true> cr;
  chunk_load<D, true>(cr, qb, kb, vb, tok_stride, t_begin, a.n);
  for (int t0 = t_begin; t0 < t_end; t0 += LC) {
    __syncthreads();  // readers of the previous chunk are done
    chunk_store<D, true>(cr, sm, t0, t_end);
    __syncthreads();
    if (t0 + LC < t_end) chunk_load<D, true>(cr, qb, kb, vb, tok_stride, t0 + LC, a.n);

    // intra-chunk scores of query block ib = wave, key blocks kb <= ib
    // (plus a zero block where the next MFMA reads past the diagonal)
    const int ib = wave;
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk) {
      if (kbk > (ib | 1)) break;
      f32x4 acc = zero4();
      if (kbk <= ib) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 qa = as_bf16x8(lds_read16(&sm.q[16 * ib + r16][32 * s + 8 * g]));
          const bf16x8 kk = as_bf16x8(lds_read16(&sm.k[16 * kbk + r16][32 * s + 8 * g]));
          acc = mfma16(qa, kk, acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * g + r, j = 16 * kbk + r16;
        const uint32_t ab = j <= i ? f2bf(acc[r]) : 0u;
        sm.a[i][j] = (bf16_t)ab;
        rsum[r] += bf2f(ab);
      }
    }
    // den for the 16 rows of block ib: rowsum(A) + phi(q) . z
    {
      float qz = 0.f;
      const int i = 16 * ib + r16;
#pragma unroll
      for (int c = 0; c < D / 4; c += 8) {
        float qf[8];
        Vec<bf16_t>::load(&sm.q[i][(D / 4) * g + c], qf);
#pragma unroll
        for (int u = 0; u < 8; ++u) qz = fmaf(qf[u], sm.z[zc][(D / 4) * g + c + u], qz);
      }
      qz += __shfl_xor(qz, 16, WAVE);
      qz += __shfl_xor(qz, 32, WAVE);
#pragma unroll
      for (int r = 0; r < 4; ++r) rsum[r] = group_sum(rsum[r], 16);
      // row r16 of the block: rsum[r16 % 4] of lane group r16 / 4
      float mine = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = __shfl(rsum[r], 16 * (r16 >> 2), WAVE);
        if ((r16 & 3) == r) mine = x;
      }
      if (g == 0) sm.den[i] = mine + qz;
    }
    __syncthreads();  // A and den complete

    // num = A V + phi(Q) S for every query block and the wave's dv blocks
    uint4 shi[D / 32][NQ], slo[D / 32][NQ];
#pragma unroll
    for (int pp = 0; pp < D / 32; ++pp)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        uint32_t h8[8], l8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          split_hi_lo(S[2 * pp][q][r], h8[r], l8[r]);
          split_hi_lo(S[2 * pp + 1][q][r], h8[4 + r], l8[4 + r]);
        }
        shi[pp][q] = make_uint4(h8[0] | (h8[1] << 16), h8[2] | (h8[3] << 16), h8[4] | (h8[5] << 16),
                                h8[6] | (h8[7] << 16));
        slo[pp][q] = make_uint4(l8[0] | (l8[1] << 16), l8[2] | (l8[3] << 16), l8[4] | (l8[5] << 16),
                                l8[6] | (l8[7] << 16));
      }
#pragma unroll
    for (int ibq = 0; ibq < 4; ++ibq) {
      f32x4 num[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) num[q] = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && ibq < 2) break;
        const bf16x8 aa = as_bf16x8(lds_read16(&sm.a[16 * ibq + r16][32 * s + 8 * g]));
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const bf16x8 vv = as_bf16x8(lds_read16(&sm.vt[16 * (wave * NQ + q) + r16][32 * s + 8 * g]));
          num[q] = mfma16(aa, vv, num[q]);
        }
      }
#pragma unroll
      for (int pp = 0; pp < D / 32; ++pp) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(&sm.q[16 * ibq + r16][32 * pp + 4 * g]);
        const uint2 x1 = *reinterpret_cast<const uint2*>(&sm.q[16 * ibq + r16][32 * pp + 16 + 4 * g]);
        const bf16x8 qa = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          num[q] = mfma16(qa, as_bf16x8(shi[pp][q]), num[q]);
          num[q] = mfma16(qa, as_bf16x8(slo[pp][q]), num[q]);
        }
      }
      // outputs of rows 16 ibq + 4 g + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ibq + 4 * g + r;
        const int t = t0 + i;
        const float inv = normalized ? 1.f / sm.den[i] : 1.f;
        if (t < t_end) {
          float* o = a.o_lin + ((size_t)b * a.n + t) * tok_stride + (size_t)h * D;
#pragma unroll
          for (int q = 0; q < NQ; ++q) o[16 * (wave * NQ + q) + r16] = num[q][r] * inv;
        }
      }
    }
    // state and normaliser after the chunk
    state_update<D>(S, sm, wave);
    if (tid < D) sm.z[zc ^ 1][tid] = sm.z[zc][tid] + chunk_ksum<D>(sm, tid);
    zc ^= 1;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool linear_mfma_supported(const Shape& sh) { return sh.dtype == 1 && (sh.d == 64 || sh.d == 128); }

void linear_segments(const Shape& sh, int n, int& nseg, int& seg_len) {
  const int chunks = (n + LC - 1) / LC;
  const int bh = sh.B * sh.H_L;
  int want = (512 + bh - 1) / bh;
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
  if (a.sh.d == 128) klaunch(k_lin_seg_sums<128>, grid, dim3(LT), 0, st, a);
  else klaunch(k_lin_seg_sums<64>, grid, dim3(LT), 0, st, a);
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
  if (a.sh.d == 128) klaunch(k_lin_chunks<128>, grid, dim3(LT), 0, st, a);
  else klaunch(k_lin_chunks<64>, grid, dim3(LT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
