// Decode-step kernels of the LISA layer for gfx950.
//
// Phase A (one launch, heterogeneous blocks, all HBM-streaming):
//   * indexer tiles: ReLU dot-product scores of the new query against every
//     cached index key, summed over indexer heads ("LISA", arXiv 2607.19358v1,
//     Section 3.2 Stage 2); the tile holding the new token also appends its
//     k, v and index key to the caches;
//   * linear slices: S += phi(k)^T v, z += phi(k), and the branch output
//     phi(q) S / (phi(q) . z) for a 32-column slice of S (Section 3.3
//     Eqs. 3-4, phi = elu + 1);
//   * gate chunks: partial dot products x . W_g[:, h] over 64 hidden rows
//     (Section 3.3 Eq. 5); the attention epilogue sums them.
// Attention: gathered GQA softmax attention over the selected rows, split
//   over the selected set; each split writes its (max, sum, accumulator)
//   partial, and a separate merge launch combines the splits and applies the
//   gate epilogue out = g*O_s + (1-g)*O_L (Section 3.2 Eq. 1, with the gate
//   on the sparse branch).
#include <type_traits>

#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_attend.h"

namespace lisa {

constexpr int PA_THREADS = 256;
// Index-key rows each lane loads at once (the rows of a block's tile are
// U * rows per wave step * 4 waves), by the step's total cached rows
// B * max_len: a few long rows want many small tiles (more blocks in flight
// at once, a shorter chain per block); many rows want fewer, larger tiles.
// Measured on the Qwen-7B layer: one 16K row 23.9 -> 23.6 us per step with
// U = 2; 32 rows of 4K-16K 114.7 -> 113.2 us with U = 8 (U = 4 between).
constexpr int IDX_ROWS_SMALL = 32768;   // B * max_len at most this: U = 2
constexpr int IDX_ROWS_LARGE = 262144;  // at least this: U = 8
inline int index_rows_in_flight(const Shape& sh) {
  const size_t rows = (size_t)sh.B * sh.max_len;
  return rows <= (size_t)IDX_ROWS_SMALL ? 2 : rows >= (size_t)IDX_ROWS_LARGE ? 8 : 4;
}
constexpr int LIN_COLS = 32;     // columns of S per linear block
constexpr int GATE_ROWS = 64;    // hidden rows per gate block

// ---------------------------------------------------------------------------
// cache append of the new token (row L-1): k, v, and the index key when the
// indexer runs
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void append_row(const PhaseAArgs& a, int b, int L) {
  constexpr int VEC = Vec<T>::N;
  const Shape& sh = a.sh;
  const size_t row = (size_t)b * sh.cap + (L - 1);
  if (a.k_idx_new && a.k_idx_cache) {
    const int E = sh.H_Ik * sh.d_I;
    T* kic = (T*)a.k_idx_cache + row * E;
    const T* kin = (const T*)a.k_idx_new + (size_t)b * E;
    for (int e = threadIdx.x * VEC; e < E; e += PA_THREADS * VEC)
      *reinterpret_cast<uint4*>(kic + e) = *reinterpret_cast<const uint4*>(kin + e);
  }
  const int EK = sh.H_kv * sh.d;
  T* kcd = (T*)a.k_cache + row * EK;
  T* vcd = (T*)a.v_cache + row * EK;
  const T* kn = (const T*)a.k_new + (size_t)b * EK;
  const T* vn = (const T*)a.v_new + (size_t)b * EK;
  for (int e = threadIdx.x * VEC; e < EK; e += PA_THREADS * VEC) {
    *reinterpret_cast<uint4*>(kcd + e) = *reinterpret_cast<const uint4*>(kn + e);
    *reinterpret_cast<uint4*>(vcd + e) = *reinterpret_cast<const uint4*>(vn + e);
  }
}

// Without scoring (sliding window): one block per sequence appends the new
// token and writes the window's index list.
template <typename T>
__device__ __forceinline__ void append_block(const PhaseAArgs& a, int b) {
  const int L = a.seq_lens[b];
  if (a.append) append_row<T>(a, b, L);
  if (a.window_idx) {
    const int m = min(a.M, L);
    for (int k = threadIdx.x; k < a.M; k += PA_THREADS) a.window_idx[(size_t)b * a.M + k] = k < m ? L - m + k : -1;
  }
}

// ---------------------------------------------------------------------------
// indexer tile
// ---------------------------------------------------------------------------
template <typename T, int R, int U>
__device__ __forceinline__ void index_tile(const PhaseAArgs& a, int b, int tile, int tile_rows) {
  using V = Vec<T>;
  constexpr int VEC = V::N;
  const Shape& sh = a.sh;
  const int L = a.seq_lens[b];
  const int j0 = tile * tile_rows;
  if (j0 >= L) return;
  const int j1 = min(L, j0 + tile_rows);
  const int E = sh.H_Ik * sh.d_I;
  const int LPR = E / VEC;       // lanes per row
  const int LPH = sh.d_I / VEC;  // lanes per key head
  const int RPW = WAVE / LPR;    // rows per wave step
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int rw = lane / LPR, li = lane % LPR;
  const int e0 = li * VEC;
  const int kh = e0 / sh.d_I, c0 = e0 % sh.d_I;
  const int step = RPW * (PA_THREADS / WAVE);  // tile_rows == U * step

  const T* kc = (const T*)a.k_idx_cache + (size_t)b * sh.cap * E;
  const T* knew = (const T*)a.k_idx_new + (size_t)b * E;
  // every lane loads U rows at once; rows past the tile end re-read the last
  // row (no branch around the loads, so they are all in flight together)
  float kv[U][VEC];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = min(j0 + u * step + wave * RPW + rw, j1 - 1);
    const T* src = (j == L - 1 && a.k_idx_new) ? knew : kc + (size_t)j * E;
    V::load(src + e0, kv[u]);
  }
  float qv[R][VEC];
  float wv[R];
  const T* qb = (const T*)a.q_idx + (size_t)b * sh.H_I * sh.d_I;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = kh * R + r;
    V::load(qb + (size_t)h * sh.d_I + c0, qv[r]);
    wv[r] = a.w_idx[h];
  }
  float* srow = a.scores + (size_t)b * a.scores_ld;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) dot = fmaf(qv[r][v], kv[u][v], dot);
      dot = group_sum(dot, LPH);
      sc = fmaf(wv[r], fmaxf(dot, 0.f), sc);
    }
    // sum over the key heads of the row (values are uniform per head group)
    sc = group_sum_range(sc, LPH, LPR);
    const int j = j0 + u * step + wave * RPW + rw;
    if (li == 0 && j < j1) srow[j] = sc;
  }

  // append the new token (the tile that holds row L-1)
  if (a.append && j0 <= L - 1 && L - 1 < j1) append_row<T>(a, b, L);
}

// ---------------------------------------------------------------------------
// linear state slice: 32 columns of S for one (sequence, head)
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void linear_slice(const PhaseAArgs& a, int b, int h, int slice) {
  // Every slice reads phi(k) and phi(q); only slice 0 reads and rewrites z
  // and forms the denominator phi(q) . z_new, so no block reads a z that
  // another block of the same launch has already advanced.  The numerator
  // phi(q) S_new of the slice's columns goes to o_lin; the epilogue divides.
  constexpr int NF = 4;  // float4 of S per thread: d * 8 / 256 <= 4 for d <= 128
  __shared__ float fk[128], fq[128], fq_z[128], vv[LIN_COLS], red[PA_THREADS / WAVE][LIN_COLS];
  const Shape& sh = a.sh;
  const int d = sh.d;
  const int c0 = slice * LIN_COLS;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const size_t hv = ((size_t)b * sh.H_L + h) * d;
  float* Sh = a.S + hv * d;  // [d, d]
  const int c4 = tid & 7;    // float4 column of this thread, constant over k
  // issue the S loads first; rows past d (d < 128) re-read row d-1
  float4 sv[NF];
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int row = min((tid + PA_THREADS * k) >> 3, d - 1);
    sv[k] = reinterpret_cast<const float4*>(Sh + (size_t)row * d + c0)[c4];
  }
  // the per-head vectors, loaded unconditionally (clamped) so that they are
  // in flight together with the S loads; z is only used (and rewritten) by
  // slice 0, and q only when the output is wanted
  const int ti = min(tid, d - 1);
  const float kr = ld1<T>((const T*)a.k_lin + hv + ti);
  const float qr = ld1<T>((const T*)(a.linear_output ? a.q_lin : a.k_lin) + hv + ti);
  const float zr = a.z[hv + ti];
  const float vr = ld1<T>((const T*)a.v_lin + hv + c0 + (tid & (LIN_COLS - 1)));
  if (tid < d) {
    const float k = phi(kr);
    const float q = a.linear_output ? phi(qr) : 0.f;
    fk[tid] = k;
    fq[tid] = q;
    if (slice == 0) {
      const float zn = zr + k;
      a.z[hv + tid] = zn;
      fq_z[tid] = q * zn;
    }
  }
  if (tid < LIN_COLS) vv[tid] = vr;
  __syncthreads();

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int rr = (tid + PA_THREADS * k) >> 3;
    if (rr < d) {
      float4 s = sv[k];
      const float kk = fk[rr];
      s.x = fmaf(kk, vv[c4 * 4 + 0], s.x);
      s.y = fmaf(kk, vv[c4 * 4 + 1], s.y);
      s.z = fmaf(kk, vv[c4 * 4 + 2], s.z);
      s.w = fmaf(kk, vv[c4 * 4 + 3], s.w);
      reinterpret_cast<float4*>(Sh + (size_t)rr * d + c0)[c4] = s;
      if (a.linear_output) {
        const float q = fq[rr];
        acc[0] = fmaf(q, s.x, acc[0]);
        acc[1] = fmaf(q, s.y, acc[1]);
        acc[2] = fmaf(q, s.z, acc[2]);
        acc[3] = fmaf(q, s.w, acc[3]);
      }
    }
  }
  if (!a.linear_output) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = sum_lanes_mod8(acc[k]);  // lanes with equal c4
  if (lane < 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) red[wave][lane * 4 + k] = acc[k];
  }
  if (slice == 0 && wave == 0) {
    float den = 0.f;
    for (int i = lane; i < d; i += WAVE) den += fq_z[i];
    den = group_sum(den, WAVE);
    if (lane == 0) a.lin_den[(size_t)b * sh.H_L + h] = den;
  }
  __syncthreads();
  if (tid < LIN_COLS) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < PA_THREADS / WAVE; ++w) o += red[w][tid];
    a.o_lin[hv + c0 + tid] = o;
  }
}

// ---------------------------------------------------------------------------
// gate partial dot products over 64 hidden rows
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void gate_chunk(const PhaseAArgs& a, int b, int chunk) {
  constexpr int KMAX = GATE_ROWS / 4;  // rows per thread for 64 head lanes x 4 row groups
  __shared__ float gred[PA_THREADS];
  const Shape& sh = a.sh;
  const int HP = sh.H_q <= 32 ? 32 : 64;
  const int RG = PA_THREADS / HP;
  const int tid = threadIdx.x;
  const int h = tid % HP, rg = tid / HP;
  const int r0 = chunk * GATE_ROWS, r1 = min(sh.hidden, r0 + GATE_ROWS);
  const int hc = min(h, sh.H_q - 1);
  const T* x = (const T*)a.x + (size_t)b * sh.hidden;
  const T* w = (const T*)a.w_gate;
  // all loads first (rows past the chunk re-read its last row), then the sum
  float xv[KMAX], wv[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int r = min(r0 + rg + RG * k, r1 - 1);
    xv[k] = ld1<T>(x + r);
    wv[k] = ld1<T>(w + (size_t)r * sh.H_q + hc);
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (r0 + rg + RG * k < r1) acc = fmaf(xv[k], wv[k], acc);
  gred[tid] = acc;
  __syncthreads();
  if (tid < sh.H_q) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += gred[g * HP + tid];
    a.gate_part[((size_t)b * a.gate_chunks + chunk) * sh.H_q + tid] = s;
  }
}

template <typename T, int R, int U>
__global__ __launch_bounds__(PA_THREADS) void k_decode_phase_a(PhaseAArgs a, int n_idx, int tiles_per_seq,
                                                               int tile_rows, int n_lin, int slices) {
  int blk = blockIdx.x;
  if (blk < n_idx) {
    index_tile<T, R, U>(a, blk / tiles_per_seq, blk % tiles_per_seq, tile_rows);
    return;
  }
  blk -= n_idx;
  if (!a.do_scores && (a.append || a.window_idx)) {  // no index tiles: one append block per sequence
    if (blk < a.sh.B) {
      append_block<T>(a, blk);
      return;
    }
    blk -= a.sh.B;
  }
  if (blk < n_lin) {
    const int per_b = a.sh.H_L * slices;
    const int b = blk / per_b, rem = blk % per_b;
    linear_slice<T>(a, b, rem / slices, rem % slices);
    return;
  }
  blk -= n_lin;
  gate_chunk<T>(a, blk / a.gate_chunks, blk % a.gate_chunks);
}

template <typename T, int R, int U>
static hipError_t launch_pa(const PhaseAArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  const int VEC = Vec<T>::N;
  const int tile_rows = U * (WAVE / (sh.H_Ik * sh.d_I / VEC)) * (PA_THREADS / WAVE);
  const int tiles = a.do_scores ? (sh.max_len + tile_rows - 1) / tile_rows : 0;
  const int n_idx = tiles * sh.B;
  const int slices = sh.d / LIN_COLS;
  const int n_lin = a.do_linear ? sh.B * sh.H_L * slices : 0;
  const int n_gate = a.do_gate ? sh.B * a.gate_chunks : 0;
  const int n_app = (!a.do_scores && (a.append || a.window_idx)) ? sh.B : 0;
  const int grid = n_idx + n_app + n_lin + n_gate;
  if (grid == 0) return hipSuccess;
  klaunch((k_decode_phase_a<T, R, U>), dim3(grid), dim3(PA_THREADS), 0, st, a, n_idx, tiles, tile_rows,
                     n_lin, slices);
  return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_pa_r(const PhaseAArgs& a, hipStream_t st) {
  switch (index_rows_in_flight(a.sh)) {
    case 2: return launch_pa<T, R, 2>(a, st);
    case 8: return launch_pa<T, R, 8>(a, st);
    default: return launch_pa<T, R, 4>(a, st);
  }
}

hipError_t launch_decode_phase_a(const PhaseAArgs& a, hipStream_t st) {
  const int R = a.sh.H_I / a.sh.H_Ik;
  if (a.sh.dtype == 0) {
    if (R == 1) return launch_pa_r<float, 1>(a, st);
    if (R == 2) return launch_pa_r<float, 2>(a, st);
    return launch_pa_r<float, 4>(a, st);
  }
  if (R == 1) return launch_pa_r<bf16_t, 1>(a, st);
  if (R == 2) return launch_pa_r<bf16_t, 2>(a, st);
  return launch_pa_r<bf16_t, 4>(a, st);
}

size_t attention_partial_floats(const Shape& sh, int n_rows, int nsplit) {
  const int G = sh.H_q / sh.H_kv;
  return (size_t)n_rows * sh.H_kv * nsplit * (size_t)(G * sh.d + 2 * G);
}


template <typename T, int D, int GT>
__global__ __launch_bounds__(AT_THREADS) void k_attention(AttnArgs a) {
  constexpr bool MF = sizeof(T) == 2;  // bf16: MFMA split attention
  using SharedT = typename std::conditional<MF, AttnMfmaShared<D, GT, AT_THREADS / WAVE>,
                                            AttnMergeShared<AT_THREADS / WAVE, GT, D>>::type;
  __shared__ SharedT ms;
  const Shape& sh = a.sh;
  int blk = blockIdx.x;
  const int s = blk % a.nsplit;
  blk /= a.nsplit;
  const int g = blk % sh.H_kv;
  const int r = blk / sh.H_kv;
  const int b = r / a.rows_per_seq, t = r % a.rows_per_seq;
  const int len = a.prefill ? t + 1 : a.seq_lens[b];
  const int m = a.dense ? len : min(sh.M, len);
  const int i0 = s * a.split_len;
  if (i0 >= m) return;  // empty split: the combine skips it
  const int i1 = min(m, i0 + a.split_len);
  const int32_t* irow = (a.dense || a.window) ? nullptr : a.idx + (size_t)r * a.idx_ld;
  const int base = a.window ? len - m : 0;  // the window's first position
  auto pos_of = [irow, base](int i) { return irow ? irow[i] : base + i; };
  if constexpr (MF) attend_split_mfma<D, GT, AT_THREADS, AT_THREADS / WAVE>(a, r, g, s, len, i0, i1, pos_of, ms);
  else attend_split<T, D, GT, AT_THREADS, AT_RP>(a, r, g, s, len, i0, i1, pos_of, ms);
}

// Merge the split partials of one (row, query head) and apply the epilogue.
// Lane sp of every wave loads split sp's max and sum (vector loads; the
// values are block-uniform and would otherwise become serialized scalar
// loads); every thread loads its dimension of all split accumulators at once,
// NS of them, the launch's split count rounded up to 8, 16 or 32.
template <typename T, int NS>
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  static_assert(NS <= AT_MAX_SPLITS && AT_MAX_SPLITS <= WAVE, "one lane per split");
  const Shape& sh = a.sh;
  const int D = sh.d;
  const int G = sh.H_q / sh.H_kv;
  const int h = blockIdx.x % sh.H_q;
  const int r = blockIdx.x / sh.H_q;
  const int g = h / G, hh = h % G;
  const int b = r / a.rows_per_seq, t = r % a.rows_per_seq;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int dim = min(tid, D - 1);
  const int GD = G * D, PS = GD + 2 * G;
  const size_t oi = ((size_t)r * sh.H_q + h) * D + dim;
  // Every load is issued before the row length arrives: the partials of all
  // nsplit splits (those past the row's valid splits are masked below), the
  // gate partials and the linear output.
  const int len = a.prefill ? t + 1 : a.seq_lens[b];
  const float* p0 = a.part + ((size_t)r * sh.H_kv + g) * a.nsplit * PS;
  float ov[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) ov[sp] = p0[(size_t)min(sp, a.nsplit - 1) * PS + hh * D + dim];
  const int ls = min(lane, a.nsplit - 1);
  const float m_raw = p0[(size_t)ls * PS + GD + hh];
  const float l_raw = p0[(size_t)ls * PS + GD + G + hh];
  float g_l = 0.f, ol = 0.f, den = 1.f;
  if (a.gate_part) {
    const float* gp = a.gate_part + (size_t)r * a.gate_chunks * sh.H_q + h;
    const float g0 = gp[(size_t)min(lane, a.gate_chunks - 1) * sh.H_q];
    const float g1 = gp[(size_t)min(lane + WAVE, a.gate_chunks - 1) * sh.H_q];
    g_l = (lane < a.gate_chunks ? g0 : 0.f) + (lane + WAVE < a.gate_chunks ? g1 : 0.f);
    for (int c = lane + 2 * WAVE; c < a.gate_chunks; c += WAVE) g_l += gp[(size_t)c * sh.H_q];
    ol = a.o_lin[oi];
    if (a.lin_den) den = a.lin_den[(size_t)r * sh.H_q + h];
  }
  const int m = a.dense ? len : min(sh.M, len);
  const int nvalid = (m + a.split_len - 1) / a.split_len;
  const bool live = lane < nvalid;
  const float mx = group_max(live ? m_raw : -INFINITY, WAVE);
  const float f_l = live ? scale_from(m_raw, mx) : 0.f;  // weight of split `lane`
  const float l = group_sum(live ? l_raw * f_l : 0.f, WAVE);
  float o = 0.f;
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f_l), sp));
    o = fmaf(sp < nvalid ? ov[sp] : 0.f, f, o);  // stale partials past the row never enter
  }
  const float gsum = group_sum(g_l, WAVE);  // every lane of the wave takes part
  if (tid >= D) return;
  o = o / l;
  if (a.gate_part) {
    const float gv = sigmoidf(gsum);
    o = gv * o + (1.f - gv) * (ol / den);
  }
  st1<T>((T*)a.out + oi, o);
}

template <typename T, int D>
static hipError_t launch_attn_td(const AttnArgs& a, dim3 grid, hipStream_t st) {
  const int G = a.sh.H_q / a.sh.H_kv;
  if (G <= 2) klaunch((k_attention<T, D, 2>), grid, dim3(AT_THREADS), 0, st, a);
  else if (G <= 4) klaunch((k_attention<T, D, 4>), grid, dim3(AT_THREADS), 0, st, a);
  else if (G <= 5) klaunch((k_attention<T, D, 5>), grid, dim3(AT_THREADS), 0, st, a);
  else if (G <= 7) klaunch((k_attention<T, D, 7>), grid, dim3(AT_THREADS), 0, st, a);
  else klaunch((k_attention<T, D, 8>), grid, dim3(AT_THREADS), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  if (a.nsplit > AT_MAX_SPLITS) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)a.n_rows * a.sh.H_kv * a.nsplit));
  switch (a.sh.d) {
    case 32: return launch_attn_td<T, 32>(a, grid, st);
    case 64: return launch_attn_td<T, 64>(a, grid, st);
    case 128: return launch_attn_td<T, 128>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_combine_t(const AttnArgs& a, hipStream_t st) {
  if (a.nsplit == 1) return hipSuccess;
  const dim3 grid((unsigned)((size_t)a.n_rows * a.sh.H_q));
  if (a.nsplit <= 8) klaunch((k_attn_combine<T, 8>), grid, dim3(128), 0, st, a);
  else if (a.nsplit <= 16) klaunch((k_attn_combine<T, 16>), grid, dim3(128), 0, st, a);
  else klaunch((k_attn_combine<T, AT_MAX_SPLITS>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  return a.sh.dtype == 0 ? launch_attn_t<float>(a, st) : launch_attn_t<bf16_t>(a, st);
}

hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t st) {
  return a.sh.dtype == 0 ? launch_combine_t<float>(a, st) : launch_combine_t<bf16_t>(a, st);
}

}  // namespace lisa
