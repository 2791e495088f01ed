// Indexer training objective ("LISA", arXiv 2607.19358v1, Section 3.2
// Stage 2, Eq. 2): for every prefill row t and indexer head j,
//   KL[t, j] = sum_{k<=t} T_k (ln T_k - ln Q_k),
// where Q = softmax of head j's ReLU score row S_k = max(0, q_I[t,j].k_I[k])
// (no head weight) and T is the mean of the causal softmax rows of the G_T =
// H_q / H_I teacher heads j G_T .. (j+1) G_T - 1 (scale 1/sqrt(d)).  With
// ln Q_k = S_k - lse(S) and sum_k T_k = 1,
//   KL = sum_k T_k ln T_k - sum_k T_k S_k + lse(S) sum_k T_k,
// so each row needs every teacher head's log-sum-exp before T can be
// formed: two passes over the row's keys.
//
//  * bf16, d = 128, d_I = 64, teacher group inside one KV head: MFMA.  A
//    wave owns 16 rows of one indexer head and holds those rows of the G_T
//    teacher heads and of the index head as MFMA B operands; the block's
//    four waves take 64 consecutive rows and share 64-key tiles of K and k_I
//    staged in LDS (double-buffered, one barrier per tile).  Per 16-key
//    sub-tile a lane gets four keys of its row for every head.  Pass 1 keeps
//    a running (max, sum of exp) per head and lane, merged over the row's
//    four lanes at the end; pass 2 forms T and accumulates the three sums.
//  * every other shape: one block per (row, head) on the vector units.
#include <math.h>

#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"

namespace lisa {

constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.44269504088896341f;

// running (max, sum of exp2) of base-2 logits; masked keys enter as -inf
__device__ __forceinline__ void online4(float& m, float& s, float v0, float v1, float v2, float v3) {
  const float mn = fmaxf(fmaxf(m, fmaxf(v0, v1)), fmaxf(v2, v3));
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(v0 - mn) + __builtin_amdgcn_exp2f(v1 - mn) +
      __builtin_amdgcn_exp2f(v2 - mn) + __builtin_amdgcn_exp2f(v3 - mn);
  m = mn;
}

__device__ __forceinline__ void merge2_xor(float& m, float& s, int mask) {
  const float m2 = __shfl_xor(m, mask, WAVE), s2 = __shfl_xor(s, mask, WAVE);
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

template <int D, int DI, int GT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_kl_mfma(KlArgs a) {
  constexpr int KT = 64, KP = D + 8, IP = DI + 8;
  __shared__ bf16_t sk[2][KT][KP];
  __shared__ bf16_t si[2][KT][IP];
  const Shape& sh = a.sh;
  const int n = a.n;
  const int nrb = (n + 63) / 64;
  const int R0 = 64 * (nrb - 1 - (int)blockIdx.x);  // longest rows first
  const int j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int T0 = R0 + 16 * wave;
  const int row = T0 + r16, rowc = min(row, n - 1);
  const int h0 = j * GT;
  const int kvh = h0 / (sh.H_q / sh.H_kv);
  const int jk = j * sh.H_Ik / sh.H_I;
  const bf16_t* qb = (const bf16_t*)a.q + (size_t)b * n * sh.H_q * D;
  const bf16_t* kb = (const bf16_t*)a.k_cache + (size_t)b * sh.cap * sh.H_kv * D;
  const bf16_t* qib = (const bf16_t*)a.q_idx + (size_t)b * n * sh.H_I * DI;
  const bf16_t* kib = (const bf16_t*)a.k_idx + (size_t)b * sh.cap * sh.H_Ik * DI;

  bf16x8 qf[GT][D / 32], qif[DI / 32];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      qf[h][k] = as_bf16x8(ld16(qb + ((size_t)rowc * sh.H_q + h0 + h) * D + 32 * k + 8 * g));
#pragma unroll
  for (int k = 0; k < DI / 32; ++k) qif[k] = as_bf16x8(ld16(qib + ((size_t)rowc * sh.H_I + j) * DI + 32 * k + 8 * g));

  constexpr int NK = KT * D / 8 / 256, NI = KT * DI / 8 / 256;
  static_assert(NK >= 1 && NI >= 1, "tile loads");
  uint4 rk[NK], ri[NI];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const int e = tid + 256 * m, key = e / (D / 8), c8 = e % (D / 8);
      rk[m] = ld16(kb + ((size_t)min(kt * KT + key, n - 1) * sh.H_kv + kvh) * D + 8 * c8);
    }
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int e = tid + 256 * m, key = e / (DI / 8), c8 = e % (DI / 8);
      ri[m] = ld16(kib + ((size_t)min(kt * KT + key, n - 1) * sh.H_Ik + jk) * DI + 8 * c8);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const int e = tid + 256 * m, key = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&sk[buf][key][8 * c8]) = rk[m];
    }
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int e = tid + 256 * m, key = e / (DI / 8), c8 = e % (DI / 8);
      *reinterpret_cast<uint4*>(&si[buf][key][8 * c8]) = ri[m];
    }
  };

  const int ntile = min(R0 + 63, n - 1) / KT + 1;  // key tiles up to the block's last row
  const int wlast = min(T0 + 15, n - 1);           // the wave's last row
  const float c2 = a.scale * LOG2E;                // base-2 teacher logits
  float mt[GT], st[GT], mi = -INFINITY, si_ = 0.f;
#pragma unroll
  for (int h = 0; h < GT; ++h) { mt[h] = -INFINITY; st[h] = 0.f; }
  float lt[GT], lse_s = 0.f;                       // pass-1 results: base-2 teacher lse, natural index lse
  float acc_tl = 0.f, acc_ts = 0.f, acc_t = 0.f;
#pragma unroll
  for (int h = 0; h < GT; ++h) lt[h] = 0.f;

  for (int pass = 0; pass < 2; ++pass) {
    fetch(0);
    stage(0);
    __syncthreads();
    for (int kt = 0; kt < ntile; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < ntile) fetch(kt + 1);
      const int J0 = kt * KT;
#pragma unroll 1
      for (int sb = 0; sb < 4; ++sb) {
        const int K0 = J0 + 16 * sb;
        if (K0 > wlast) break;  // wave-uniform: no key of the sub-tile is causal for the wave
        bf16x8 kf[D / 32], kif[DI / 32];
#pragma unroll
        for (int k = 0; k < D / 32; ++k) kf[k] = as_bf16x8(lds_read16(&sk[buf][16 * sb + r16][32 * k + 8 * g]));
#pragma unroll
        for (int k = 0; k < DI / 32; ++k) kif[k] = as_bf16x8(lds_read16(&si[buf][16 * sb + r16][32 * k + 8 * g]));
        f32x4 ai = zero4();
#pragma unroll
        for (int k = 0; k < DI / 32; ++k) ai = mfma16(kif[k], qif[k], ai);
        f32x4 at[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          at[h] = zero4();
#pragma unroll
          for (int k = 0; k < D / 32; ++k) at[h] = mfma16(kf[k], qf[h][k], at[h]);
        }
        // lane: keys K0 + 4 g + e of row `row`
        const int kk = K0 + 4 * g;
        bool ok[4];
        float S[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[e] = kk + e <= row && row < n;
          S[e] = fmaxf(ai[e], 0.f);
        }
        if (pass == 0) {
          online4(mi, si_, ok[0] ? S[0] * LOG2E : -INFINITY, ok[1] ? S[1] * LOG2E : -INFINITY,
                  ok[2] ? S[2] * LOG2E : -INFINITY, ok[3] ? S[3] * LOG2E : -INFINITY);
#pragma unroll
          for (int h = 0; h < GT; ++h)
            online4(mt[h], st[h], ok[0] ? at[h][0] * c2 : -INFINITY, ok[1] ? at[h][1] * c2 : -INFINITY,
                    ok[2] ? at[h][2] * c2 : -INFINITY, ok[3] ? at[h][3] * c2 : -INFINITY);
        } else {
          float T[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) T[e] += __builtin_amdgcn_exp2f(fmaf(at[h][e], c2, -lt[h]));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = T[e] * (1.f / GT);
            if (ok[e]) {
              if (t > 1e-30f) acc_tl = fmaf(t, __builtin_amdgcn_logf(t) * LN2, acc_tl);  // t ln t; smaller t add < 1e-28
              acc_ts = fmaf(t, S[e], acc_ts);
              acc_t += t;
            }
          }
        }
      }
      if (kt + 1 < ntile) stage(buf ^ 1);
      __syncthreads();
    }
    if (pass == 0) {  // merge the row's four lanes (g), then fix the normalisers
      merge2_xor(mi, si_, 16);
      merge2_xor(mi, si_, 32);
      lse_s = (mi + __builtin_amdgcn_logf(si_)) * LN2;
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        merge2_xor(mt[h], st[h], 16);
        merge2_xor(mt[h], st[h], 32);
        lt[h] = mt[h] + __builtin_amdgcn_logf(st[h]);
      }
    }
  }
  acc_tl += __shfl_xor(acc_tl, 16, WAVE);
  acc_tl += __shfl_xor(acc_tl, 32, WAVE);
  acc_ts += __shfl_xor(acc_ts, 16, WAVE);
  acc_ts += __shfl_xor(acc_ts, 32, WAVE);
  acc_t += __shfl_xor(acc_t, 16, WAVE);
  acc_t += __shfl_xor(acc_t, 32, WAVE);
  if (g == 0 && row < n) a.kl[((size_t)b * n + row) * sh.H_I + j] = acc_tl - acc_ts + lse_s * acc_t;
}

// Any shape: one block per (row, indexer head); per-thread log-sum-exp
// pairs over a stride of keys, merged over the block.
template <typename T>
__global__ __launch_bounds__(256) void k_kl_valu(KlArgs a) {
  __shared__ float rm[4], rs[4], red[4];
  __shared__ float lse_t[64];
  const Shape& sh = a.sh;
  const int n = a.n, t = blockIdx.x, j = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int GTr = sh.H_q / sh.H_I, h0 = j * GTr, G = sh.H_q / sh.H_kv;
  const int jk = j * sh.H_Ik / sh.H_I;
  const int d = sh.d, dI = sh.d_I;
  const T* qi = (const T*)a.q_idx + (((size_t)b * n + t) * sh.H_I + j) * dI;
  const T* kib = (const T*)a.k_idx + (size_t)b * sh.cap * sh.H_Ik * dI;
  const T* qb = (const T*)a.q + ((size_t)b * n + t) * sh.H_q * d;
  const T* kb = (const T*)a.k_cache + (size_t)b * sh.cap * sh.H_kv * d;
  auto dot = [&](const T* x, const T* y, int len) {
    float s = 0.f;
    for (int c = 0; c < len; ++c) s = fmaf(ld1(x + c), ld1(y + c), s);
    return s;
  };
  auto score = [&](int k) { return fmaxf(dot(qi, kib + ((size_t)k * sh.H_Ik + jk) * dI, dI), 0.f); };
  auto logit = [&](int h, int k) { return dot(qb + (size_t)h * d, kb + ((size_t)k * sh.H_kv + h / G) * d, d) * a.scale; };
  auto block_lse = [&](float m, float s) {  // merge the block's pairs; natural-log lse
#pragma unroll
    for (int mask = 1; mask < WAVE; mask <<= 1) lse_merge_xor(m, s, mask);
    if ((tid & (WAVE - 1)) == 0) { rm[tid / WAVE] = m; rs[tid / WAVE] = s; }
    __syncthreads();
    m = rm[0]; s = rs[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(m, s, rm[w], rs[w]);
    __syncthreads();
    return m + logf(s);
  };
  float m = -INFINITY, s = 0.f;
  for (int k = tid; k <= t; k += 256) lse_merge(m, s, score(k), 1.f);
  const float lse_s = block_lse(m, s);
  for (int h = 0; h < GTr; ++h) {
    m = -INFINITY; s = 0.f;
    for (int k = tid; k <= t; k += 256) lse_merge(m, s, logit(h0 + h, k), 1.f);
    const float l = block_lse(m, s);
    if (tid == 0) lse_t[h] = l;
  }
  __syncthreads();
  float acc_tl = 0.f, acc_ts = 0.f, acc_t = 0.f;
  for (int k = tid; k <= t; k += 256) {
    float tk = 0.f;
    for (int h = 0; h < GTr; ++h) tk += expf(logit(h0 + h, k) - lse_t[h]);
    tk /= (float)GTr;
    if (tk > 1e-30f) acc_tl = fmaf(tk, logf(tk), acc_tl);
    acc_ts = fmaf(tk, score(k), acc_ts);
    acc_t += tk;
  }
  acc_tl = block_sum256(acc_tl, red);
  acc_ts = block_sum256(acc_ts, red);
  acc_t = block_sum256(acc_t, red);
  if (tid == 0) a.kl[((size_t)b * n + t) * sh.H_I + j] = acc_tl - acc_ts + lse_s * acc_t;
}

// Loss of Eq. 2: the mean of every KL value (one block of 1024 threads,
// four values in flight per thread, a fixed summation order).
__global__ __launch_bounds__(1024) void k_kl_loss(KlArgs a, int count) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i0 = threadIdx.x; i0 < count; i0 += 4096) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + 1024 * u < count ? a.kl[i0 + 1024 * u] : 0.f;
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  s = group_sum(s, WAVE);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += red[w];
    a.loss[0] = t / (float)count;
  }
}

bool kl_mfma_supported(const Shape& sh) {
  const int GT = sh.H_q / sh.H_I, G = sh.H_q / sh.H_kv;
  return sh.dtype == 1 && sh.d == 128 && sh.d_I == 64 && GT >= 1 && GT <= 8 && G % GT == 0;
}

hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (kl_mfma_supported(sh)) {
    const dim3 grid((unsigned)((a.n + 63) / 64), (unsigned)sh.H_I, (unsigned)sh.B);
    switch (sh.H_q / sh.H_I) {
      case 1: klaunch((k_kl_mfma<128, 64, 1>), grid, dim3(256), 0, st, a); break;
      case 2: klaunch((k_kl_mfma<128, 64, 2>), grid, dim3(256), 0, st, a); break;
      case 3: klaunch((k_kl_mfma<128, 64, 3>), grid, dim3(256), 0, st, a); break;
      case 4: klaunch((k_kl_mfma<128, 64, 4>), grid, dim3(256), 0, st, a); break;
      case 5: klaunch((k_kl_mfma<128, 64, 5>), grid, dim3(256), 0, st, a); break;
      case 6: klaunch((k_kl_mfma<128, 64, 6>), grid, dim3(256), 0, st, a); break;
      case 7: klaunch((k_kl_mfma<128, 64, 7>), grid, dim3(256), 0, st, a); break;
      default: klaunch((k_kl_mfma<128, 64, 8>), grid, dim3(256), 0, st, a); break;
    }
  } else {
    const dim3 grid((unsigned)a.n, (unsigned)sh.H_I, (unsigned)sh.B);
    if (sh.dtype == 1) klaunch(k_kl_valu<bf16_t>, grid, dim3(256), 0, st, a);
    else klaunch(k_kl_valu<float>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_kl_loss(const KlArgs& a, hipStream_t st) {
  klaunch(k_kl_loss, dim3(1), dim3(1024), 0, st, a, a.sh.B * a.n * a.sh.H_I);
  return hipGetLastError();
}

}  // namespace lisa
