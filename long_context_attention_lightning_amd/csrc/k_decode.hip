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
//   * gate chunks: partial dot products x . W_g[:, h] over 256 hidden rows
//     (Section 3.3 Eq. 5); the attention epilogue sums them.
// Attention: gathered GQA softmax attention over the selected rows, split
//   over the selected set, with an in-kernel combine by the last split block
//   and the gate epilogue out = g*O_s + (1-g)*O_L (Section 3.2 Eq. 1, with
//   the gate on the sparse branch).
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

constexpr int PA_THREADS = 256;
constexpr int IDX_TILE = 64;     // positions per indexer block
constexpr int LIN_COLS = 32;     // columns of S per linear block
constexpr int GATE_ROWS = 256;   // hidden rows per gate block

// ---------------------------------------------------------------------------
// indexer tile
// ---------------------------------------------------------------------------
template <typename T, int R>
__device__ __forceinline__ void index_tile(const PhaseAArgs& a, int b, int tile) {
  using V = Vec<T>;
  constexpr int VEC = V::N;
  constexpr int U = 4;  // rows in flight per lane
  const Shape& sh = a.sh;
  const int L = a.seq_lens[b];
  const int j0 = tile * IDX_TILE;
  if (j0 >= L) return;
  const int j1 = min(L, j0 + IDX_TILE);
  const int E = sh.H_Ik * sh.d_I;
  const int LPR = E / VEC;       // lanes per row
  const int LPH = sh.d_I / VEC;  // lanes per key head
  const int RPW = WAVE / LPR;    // rows per wave step
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int rw = lane / LPR, li = lane % LPR;
  const int e0 = li * VEC;
  const int kh = e0 / sh.d_I, c0 = e0 % sh.d_I;

  float qv[R][VEC];
  float wv[R];
  const T* qb = (const T*)a.q_idx + (size_t)b * sh.H_I * sh.d_I;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = kh * R + r;
    V::load(qb + (size_t)h * sh.d_I + c0, qv[r]);
    wv[r] = a.w_idx[h];
  }
  const T* kc = (const T*)a.k_idx_cache + (size_t)b * sh.cap * E;
  const T* knew = (const T*)a.k_idx_new + (size_t)b * E;
  float* srow = a.scores + (size_t)b * a.scores_ld;
  const int step = RPW * (PA_THREADS / WAVE);

  for (int base = j0; base < j1; base += U * step) {
    float kv[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * step + wave * RPW + rw;
      if (j < j1) {
        const T* src = (j == L - 1 && a.k_idx_new) ? knew : kc + (size_t)j * E;
        V::load(src + e0, kv[u]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) kv[u][v] = 0.f;
      }
    }
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
      // sum over key heads: lanes li, li+LPH, ... of the row group
      for (int off = LPH; off < LPR; off <<= 1) sc += __shfl_xor(sc, off, WAVE);
      const int j = base + u * step + wave * RPW + rw;
      if (li == 0 && j < j1) srow[j] = sc;
    }
  }

  // append the new token (the tile that holds row L-1)
  if (a.append && j0 <= L - 1 && L - 1 < j1) {
    const size_t row = (size_t)b * sh.cap + (L - 1);
    T* kic = (T*)a.k_idx_cache + row * E;
    const T* kin = knew;
    for (int e = threadIdx.x * VEC; e < E; e += PA_THREADS * VEC)
      *reinterpret_cast<uint4*>(kic + e) = *reinterpret_cast<const uint4*>(kin + e);
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
  __shared__ float fk[256], fq[256], fq_z[256], vv[LIN_COLS], red[PA_THREADS / WAVE][LIN_COLS];
  const Shape& sh = a.sh;
  const int d = sh.d;
  const int c0 = slice * LIN_COLS;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const size_t hv = ((size_t)b * sh.H_L + h) * d;
  for (int i = tid; i < d; i += PA_THREADS) {
    const float k = phi(ld1<T>((const T*)a.k_lin + hv + i));
    fk[i] = k;
    float q = 0.f;
    if (a.linear_output) {
      q = phi(ld1<T>((const T*)a.q_lin + hv + i));
      fq[i] = q;
    }
    if (slice == 0) {
      const float zn = a.z[hv + i] + k;
      a.z[hv + i] = zn;
      fq_z[i] = q * zn;
    }
  }
  if (tid < LIN_COLS) vv[tid] = ld1<T>((const T*)a.v_lin + hv + c0 + tid);
  __syncthreads();

  float* Sh = a.S + hv * d;  // [d, d]
  const int c4 = tid & 7;    // float4 column of this thread, constant over f
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int f = tid; f < d * 8; f += PA_THREADS) {
    const int row = f >> 3;
    float4* p = reinterpret_cast<float4*>(Sh + (size_t)row * d + c0) + c4;
    float4 s = *p;
    const float k = fk[row];
    s.x = fmaf(k, vv[c4 * 4 + 0], s.x);
    s.y = fmaf(k, vv[c4 * 4 + 1], s.y);
    s.z = fmaf(k, vv[c4 * 4 + 2], s.z);
    s.w = fmaf(k, vv[c4 * 4 + 3], s.w);
    *p = s;
    if (a.linear_output) {
      const float q = fq[row];
      acc[0] = fmaf(q, s.x, acc[0]);
      acc[1] = fmaf(q, s.y, acc[1]);
      acc[2] = fmaf(q, s.z, acc[2]);
      acc[3] = fmaf(q, s.w, acc[3]);
    }
  }
  if (!a.linear_output) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[k] += __shfl_xor(acc[k], 8, WAVE);
    acc[k] += __shfl_xor(acc[k], 16, WAVE);
    acc[k] += __shfl_xor(acc[k], 32, WAVE);
  }
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
// gate partial dot products over 256 hidden rows
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void gate_chunk(const PhaseAArgs& a, int b, int chunk) {
  __shared__ float gred[PA_THREADS];
  const Shape& sh = a.sh;
  const int HP = sh.H_q <= 32 ? 32 : 64;
  const int RG = PA_THREADS / HP;
  const int tid = threadIdx.x;
  const int h = tid % HP, rg = tid / HP;
  const int r0 = chunk * GATE_ROWS, r1 = min(sh.hidden, r0 + GATE_ROWS);
  const T* x = (const T*)a.x + (size_t)b * sh.hidden;
  const T* w = (const T*)a.w_gate;
  float acc = 0.f;
  if (h < sh.H_q) {
#pragma unroll 8
    for (int r = r0 + rg; r < r1; r += RG) acc = fmaf(ld1<T>(x + r), ld1<T>(w + (size_t)r * sh.H_q + h), acc);
  }
  gred[tid] = acc;
  __syncthreads();
  if (tid < sh.H_q) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += gred[g * HP + tid];
    a.gate_part[((size_t)b * a.gate_chunks + chunk) * sh.H_q + tid] = s;
  }
}

template <typename T, int R>
__global__ __launch_bounds__(PA_THREADS) void k_decode_phase_a(PhaseAArgs a, int n_idx, int tiles_per_seq,
                                                               int n_lin, int slices) {
  if (blockIdx.x == 0 && a.counters) {
    for (int i = threadIdx.x; i < a.n_counters; i += PA_THREADS) a.counters[i] = 0u;
  }
  int blk = blockIdx.x;
  if (blk < n_idx) {
    index_tile<T, R>(a, blk / tiles_per_seq, blk % tiles_per_seq);
    return;
  }
  blk -= n_idx;
  if (blk < n_lin) {
    const int per_b = a.sh.H_L * slices;
    const int b = blk / per_b, rem = blk % per_b;
    linear_slice<T>(a, b, rem / slices, rem % slices);
    return;
  }
  blk -= n_lin;
  gate_chunk<T>(a, blk / a.gate_chunks, blk % a.gate_chunks);
}

template <typename T, int R>
static hipError_t launch_pa(const PhaseAArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  const int tiles = a.do_scores ? (sh.max_len + IDX_TILE - 1) / IDX_TILE : 0;
  const int n_idx = tiles * sh.B;
  const int slices = sh.d / LIN_COLS;
  const int n_lin = a.do_linear ? sh.B * sh.H_L * slices : 0;
  const int n_gate = a.do_gate ? sh.B * a.gate_chunks : 0;
  const int grid = n_idx + n_lin + n_gate;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_decode_phase_a<T, R>), dim3(grid), dim3(PA_THREADS), 0, st, a, n_idx, tiles, n_lin,
                     slices);
  return hipGetLastError();
}

hipError_t launch_decode_phase_a(const PhaseAArgs& a, hipStream_t st) {
  const int R = a.sh.H_I / a.sh.H_Ik;
  if (a.sh.dtype == 0) {
    if (R == 1) return launch_pa<float, 1>(a, st);
    if (R == 2) return launch_pa<float, 2>(a, st);
    return launch_pa<float, 4>(a, st);
  }
  if (R == 1) return launch_pa<bf16_t, 1>(a, st);
  if (R == 2) return launch_pa<bf16_t, 2>(a, st);
  return launch_pa<bf16_t, 4>(a, st);
}

// ---------------------------------------------------------------------------
// gathered GQA attention
// ---------------------------------------------------------------------------
constexpr int AT_THREADS = 256;
constexpr int GMAX = 8;       // query heads per KV head
constexpr int AT_CHUNK = 128; // positions per softmax chunk

size_t attention_partial_floats(const Shape& sh, int n_rows, int nsplit) {
  const int G = sh.H_q / sh.H_kv;
  return (size_t)n_rows * sh.H_kv * nsplit * (size_t)(G * sh.d + 2 * G);
}

template <typename T, int D>
__global__ __launch_bounds__(AT_THREADS) void k_attention(AttnArgs a) {
  using V = Vec<T>;
  constexpr int VEC = V::N;
  constexpr int LG = D / VEC;            // lanes per head row
  constexpr int NG = AT_THREADS / LG;    // position slots
  constexpr int NW = AT_THREADS / WAVE;
  __shared__ int pos[AT_CHUNK];
  __shared__ float logit[AT_CHUNK][GMAX];
  __shared__ float run_m[GMAX], run_l[GMAX], fac[GMAX];
  __shared__ float red[NW][GMAX * D];
  __shared__ int is_last;

  const Shape& sh = a.sh;
  const int G = sh.H_q / sh.H_kv;
  int blk = blockIdx.x;
  const int s = blk % a.nsplit;
  blk /= a.nsplit;
  const int g = blk % sh.H_kv;
  const int r = blk / sh.H_kv;
  const int b = r / a.rows_per_seq, t = r % a.rows_per_seq;
  const int len = a.prefill ? t + 1 : a.seq_lens[b];
  const int m = a.dense ? len : min(sh.M, len);
  const int i0 = s * a.split_len;
  if (i0 >= m) return;  // empty split: takes no part in the combine
  const int i1 = min(m, i0 + a.split_len);
  const int nvalid = (m + a.split_len - 1) / a.split_len;

  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int ps = tid / LG, li = tid % LG;
  const float scale = 1.4426950408889634f * rsqrtf((float)D);

  float q[GMAX][VEC];
  const T* qrow = (const T*)a.q + ((size_t)r * sh.H_q + (size_t)g * G) * D + li * VEC;
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh < G) {
      V::load(qrow + (size_t)hh * D, q[hh]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) q[hh][v] *= scale;
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) q[hh][v] = 0.f;
    }
  }
  float acc[GMAX][VEC];
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[hh][v] = 0.f;
  if (tid < GMAX) {
    run_m[tid] = -INFINITY;
    run_l[tid] = 0.f;
  }
  const size_t kv_b = (size_t)b * sh.cap;
  const T* kc = (const T*)a.k_cache;
  const T* vc = (const T*)a.v_cache;
  const int32_t* irow = a.idx ? a.idx + (size_t)r * a.idx_ld : nullptr;

  for (int c0 = i0; c0 < i1; c0 += AT_CHUNK) {
    const int cnt = min(AT_CHUNK, i1 - c0);
    __syncthreads();  // previous chunk fully consumed
    for (int p = tid; p < cnt; p += AT_THREADS) {
      const int pp = a.dense ? c0 + p : irow[c0 + p];
      pos[p] = min(max(pp, 0), len - 1);  // defensive: never read outside the row
    }
    __syncthreads();
    // logits
    for (int p = ps; p < cnt; p += NG) {
      float kv[VEC];
      V::load(kc + ((kv_b + pos[p]) * sh.H_kv + g) * D + li * VEC, kv);
#pragma unroll
      for (int hh = 0; hh < GMAX; ++hh) {
        if (hh < G) {
          float dot = 0.f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) dot = fmaf(q[hh][v], kv[v], dot);
          dot = group_sum(dot, LG);
          if (li == 0) logit[p][hh] = dot;
        }
      }
    }
    __syncthreads();
    // chunk max / probabilities / sums: 32 lanes per head
    {
      const int hh = tid / 32, part = tid % 32;
      if (hh < G) {
        float mx = -INFINITY;
        for (int p = part; p < cnt; p += 32) mx = fmaxf(mx, logit[p][hh]);
        mx = group_max(mx, 32);
        const float m_old = run_m[hh];
        const float m_new = fmaxf(m_old, mx);
        float sum = 0.f;
        for (int p = part; p < cnt; p += 32) {
          const float e = exp2f(logit[p][hh] - m_new);
          logit[p][hh] = e;
          sum += e;
        }
        sum = group_sum(sum, 32);
        if (part == 0) {
          const float f = exp2f(m_old - m_new);  // 0 on the first chunk
          fac[hh] = f;
          run_l[hh] = run_l[hh] * f + sum;
          run_m[hh] = m_new;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) {
      if (hh < G) {
        const float f = fac[hh];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[hh][v] *= f;
      }
    }
    for (int p = ps; p < cnt; p += NG) {
      float vv[VEC];
      V::load(vc + ((kv_b + pos[p]) * sh.H_kv + g) * D + li * VEC, vv);
#pragma unroll
      for (int hh = 0; hh < GMAX; ++hh) {
        if (hh < G) {
          const float pr = logit[p][hh];
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[hh][v] = fmaf(pr, vv[v], acc[hh][v]);
        }
      }
    }
  }
  // reduce the position slots: first inside the wave, then across waves
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh < G) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float x = acc[hh][v];
        for (int off = LG; off < WAVE; off <<= 1) x += __shfl_xor(x, off, WAVE);
        acc[hh][v] = x;
      }
    }
  }
  if (lane < LG) {
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh)
      if (hh < G)
#pragma unroll
        for (int v = 0; v < VEC; ++v) red[wave][hh * D + li * VEC + v] = acc[hh][v];
  }
  __syncthreads();

  const int GD = G * D;
  if (a.nsplit == 1) {
    for (int e = tid; e < GD; e += AT_THREADS) {
      const int hh = e / D, dim = e % D;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += red[w][e];
      o = o / run_l[hh];
      const int h = g * G + hh;
      const size_t oi = ((size_t)r * sh.H_q + h) * D + dim;
      if (a.gate_part) {
        float gl = 0.f;
        for (int c = 0; c < a.gate_chunks; ++c) gl += a.gate_part[((size_t)r * a.gate_chunks + c) * sh.H_q + h];
        const float gv = sigmoidf(gl);
        float ol = a.o_lin[oi];
        if (a.lin_den) ol = ol / a.lin_den[(size_t)r * sh.H_q + h];
        o = gv * o + (1.f - gv) * ol;
      }
      st1<T>((T*)a.out + oi, o);
    }
    return;
  }

  // split partial: unnormalised accumulator, running max and sum
  const int PS = GD + 2 * G;
  float* mypart = a.part + (((size_t)r * sh.H_kv + g) * a.nsplit + s) * PS;
  for (int e = tid; e < GD; e += AT_THREADS) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += red[w][e];
    mypart[e] = o;
  }
  if (tid < G) {
    mypart[GD + tid] = run_m[tid];
    mypart[GD + G + tid] = run_l[tid];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.counters[(size_t)r * sh.H_kv + g], 1u);
    is_last = (prev == (unsigned)(nvalid - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (tid == 0) a.counters[(size_t)r * sh.H_kv + g] = 0u;  // ready for the next call
  const float* p0 = a.part + ((size_t)r * sh.H_kv + g) * a.nsplit * PS;
  for (int e = tid; e < GD; e += AT_THREADS) {
    const int hh = e / D, dim = e % D;
    float mx = -INFINITY;
    for (int sp = 0; sp < nvalid; ++sp) mx = fmaxf(mx, p0[(size_t)sp * PS + GD + hh]);
    float l = 0.f, o = 0.f;
    for (int sp = 0; sp < nvalid; ++sp) {
      const float* ps_ = p0 + (size_t)sp * PS;
      const float f = exp2f(ps_[GD + hh] - mx);
      l = fmaf(ps_[GD + G + hh], f, l);
      o = fmaf(ps_[e], f, o);
    }
    o = o / l;
    const int h = g * G + hh;
    const size_t oi = ((size_t)r * sh.H_q + h) * D + dim;
    if (a.gate_part) {
      float gl = 0.f;
      for (int c = 0; c < a.gate_chunks; ++c) gl += a.gate_part[((size_t)r * a.gate_chunks + c) * sh.H_q + h];
      const float gv = sigmoidf(gl);
      float ol = a.o_lin[oi];
      if (a.lin_den) ol = ol / a.lin_den[(size_t)r * sh.H_q + h];
      o = gv * o + (1.f - gv) * ol;
    }
    st1<T>((T*)a.out + oi, o);
  }
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.n_rows * a.sh.H_kv * a.nsplit));
  switch (a.sh.d) {
    case 32: hipLaunchKernelGGL((k_attention<T, 32>), grid, dim3(AT_THREADS), 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_attention<T, 64>), grid, dim3(AT_THREADS), 0, st, a); break;
    case 128: hipLaunchKernelGGL((k_attention<T, 128>), grid, dim3(AT_THREADS), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  return a.sh.dtype == 0 ? launch_attn_t<float>(a, st) : launch_attn_t<bf16_t>(a, st);
}

__global__ void k_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace lisa
