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
// Block = 4 waves, one query head each, 64 query positions (4 tiles of 16)
// of one KV head; the K tile (row-major) and V tile (transposed) of 64 keys
// are staged in LDS for all four heads.  Per tile a wave computes
// S^T = K Q^T (keys along the accumulator rows, so a lane holds four
// consecutive keys of one query), masks and exponentiates it, and feeds the
// probabilities straight from registers into O += P V, with the key order
// of the contraction permuted the same way in P and in V.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"
#include "lisa_prefill.h"

namespace lisa {

constexpr int AK = 64;    // keys per tile
constexpr int AP = 4;     // query tiles of 16 per wave
constexpr int AQ = 16 * AP;

template <int D>
struct AttnShared {
  bf16_t k[AK][D + 8];
  bf16_t vt[D][AK + 8];
};

template <int D>
struct AttnRegs {
  static constexpr int NK = AK * D / 8 / 256;   // K vectors per thread
  static constexpr int NV = AK * D / 16 / 256;  // V token pairs per thread
  uint4 k[NK], v[2 * NV];
  uint2 mw[AP];                                 // mask words of the lane's query rows
};

template <int D>
__device__ __forceinline__ void attn_stage(const AttnRegs<D>& r, AttnShared<D>& sm) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
#pragma unroll
  for (int m = 0; m < AttnRegs<D>::NK; ++m) {
    const int e = tid + 256 * m;
    *reinterpret_cast<uint4*>(&sm.k[e / (D / 8)][8 * (e % (D / 8))]) = r.k[m];
  }
#pragma unroll
  for (int m = 0; m < AttnRegs<D>::NV; ++m) {
    const int tau = lane & 31, c8 = 2 * (wave + 4 * m) + (lane >> 5);
    const uint32_t a[4] = {r.v[2 * m].x, r.v[2 * m].y, r.v[2 * m].z, r.v[2 * m].w};
    const uint32_t b[4] = {r.v[2 * m + 1].x, r.v[2 * m + 1].y, r.v[2 * m + 1].z, r.v[2 * m + 1].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint32_t*>(&sm.vt[8 * c8 + 2 * e][2 * tau]) = (a[e] & 0xffffu) | (b[e] << 16);
      *reinterpret_cast<uint32_t*>(&sm.vt[8 * c8 + 2 * e + 1][2 * tau]) = (a[e] >> 16) | (b[e] & 0xffff0000u);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_attn_prefill_mfma(AttnMaskArgs a) {
  __shared__ AttnShared<D> sm;
  const Shape& sh = a.sh;
  const int G = sh.H_q / sh.H_kv;
  const int nhg = (G + 3) / 4;
  const int npb = (a.n + AQ - 1) / AQ;
  // longest causal rows first
  const int per_pb = sh.B * sh.H_kv * nhg;
  const int pb = npb - 1 - (int)(blockIdx.x / per_pb);
  int rest = blockIdx.x % per_pb;
  const int hg = rest % nhg;
  rest /= nhg;
  const int kvh = rest % sh.H_kv, b = rest / sh.H_kv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int hl = 4 * hg + wave;             // head inside the KV group
  const bool active = hl < G;               // idle waves still stage tiles
  const int h = kvh * G + min(hl, G - 1);
  const int T0 = pb * AQ;
  const int n = a.n;

  const size_t kv_stride = (size_t)sh.H_kv * D;
  const bf16_t* kb = (const bf16_t*)a.k_cache + (size_t)b * sh.cap * kv_stride + (size_t)kvh * D;
  const bf16_t* vb = (const bf16_t*)a.v_cache + (size_t)b * sh.cap * kv_stride + (size_t)kvh * D;
  const size_t q_stride = (size_t)sh.H_q * D;
  const bf16_t* qb = (const bf16_t*)a.q + (size_t)b * n * q_stride + (size_t)h * D;
  const uint32_t* mrow0 = a.mask + (size_t)b * n * a.mask_ld;

  // Q^T operands: lane holds Q[t = T0 + 16 i + r16][32 s + 8 g .. + 7]
  bf16x8 qf[AP][D / 32];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    const int t = min(T0 + 16 * i + r16, n - 1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[i][s] = as_bf16x8(ld16(qb + (size_t)t * q_stride + 32 * s + 8 * g));
  }
  f32x4 o[AP][D / 16];
#pragma unroll
  for (int i = 0; i < AP; ++i)
#pragma unroll
    for (int q = 0; q < D / 16; ++q) o[i][q] = zero4();
  float mrun[AP], lrun[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
  }
  const float scale = a.scale_log2e;
  const int tmax = min(T0 + AQ, n) - 1;
  const int nkt = tmax / AK + 1;

  // mask rows: row of query tile i for this lane, clamped to the sequence
  const uint32_t* mq = mrow0 + (size_t)min(T0, n - 1) * a.mask_ld;
  // rows past n read row n-1 (its results are never stored)
  const int mrow_clamp = n - 1 - T0;

  // next tile's K, V and mask words, held in registers while this one runs
  AttnRegs<D> rg;
  auto prefetch = [&](int J0) {
    const int tid_ = threadIdx.x, lane_ = tid_ & (WAVE - 1), wave_ = tid_ / WAVE;
#pragma unroll
    for (int m = 0; m < AttnRegs<D>::NK; ++m) {
      const int e = tid_ + 256 * m;
      const int tok = e / (D / 8), c8 = e % (D / 8);
      rg.k[m] = ld16(kb + (size_t)min(J0 + tok, n - 1) * kv_stride + 8 * c8);
    }
#pragma unroll
    for (int m = 0; m < AttnRegs<D>::NV; ++m) {
      const int tau = lane_ & 31, c8 = 2 * (wave_ + 4 * m) + (lane_ >> 5);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        rg.v[2 * m + u] = ld16(vb + (size_t)min(J0 + 2 * tau + u, n - 1) * kv_stride + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int rr = min(16 * i + (lane_ & 15), mrow_clamp);
      rg.mw[i] = *reinterpret_cast<const uint2*>(mq + (size_t)rr * a.mask_ld + J0 / 32);
    }
  };

  prefetch(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int J0 = kt * AK;
    uint2 mw[AP];
#pragma unroll
    for (int i = 0; i < AP; ++i) mw[i] = rg.mw[i];
    __syncthreads();  // readers of the previous tile are done
    attn_stage<D>(rg, sm);
    __syncthreads();
    if (kt + 1 < nkt) prefetch(J0 + AK);
    if (!active) continue;

    // K operands of the tile: key 16 c + r16, dims 32 s + 8 g .. + 7
    bf16x8 kf[4][D / 32];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kf[c][s] = as_bf16x8(lds_read16(&sm.k[16 * c + r16][32 * s + 8 * g]));

    uint4 pf[AP][2];  // probabilities as bf16, contraction order of the P V step
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int t = T0 + 16 * i + r16;
      f32x4 st[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        st[c] = zero4();
#pragma unroll
        for (int s = 0; s < D / 32; ++s) st[c] = mfma16(kf[c][s], qf[i][s], st[c]);
      }
      // lane holds s[t][J0 + 16 c + 4 g + r]
      float mt = -INFINITY;
      float sv[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t word = (c < 2) ? mw[i].x : mw[i].y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = 16 * c + 4 * g + r;
          const bool on = ((word >> ((kk & 31))) & 1u) && (J0 + kk <= t);
          sv[c][r] = on ? st[c][r] * scale : -INFINITY;
          mt = fmaxf(mt, sv[c][r]);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, WAVE));
      mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
      const float mnew = fmaxf(mrun[i], mt);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(mrun[i] - muse);
      mrun[i] = mnew;
      float lsum = 0.f;
      uint32_t pb16[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb16[c][r] = f2bf(exp2f(sv[c][r] - muse));
          lsum += bf2f(pb16[c][r]);
        }
      lrun[i] = lrun[i] * alpha + lsum;
      // contraction step s covers key blocks 2 s and 2 s + 1
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pf[i][s] = make_uint4(pb16[2 * s][0] | (pb16[2 * s][1] << 16), pb16[2 * s][2] | (pb16[2 * s][3] << 16),
                              pb16[2 * s + 1][0] | (pb16[2 * s + 1][1] << 16),
                              pb16[2 * s + 1][2] | (pb16[2 * s + 1][3] << 16));
      // rescale O rows 4 g + r by the alpha of their query (held by lane 4 g + r)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g + r, WAVE);
#pragma unroll
        for (int q = 0; q < D / 16; ++q) o[i][q][r] *= ar;
      }
    }
    // O += P V: V operand of dv block q, step s: keys {32 s + 4 g .. +3, 32 s + 16 + 4 g .. +3}
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(&sm.vt[16 * q + r16][32 * s + 4 * g]);
        const uint2 x1 = *reinterpret_cast<const uint2*>(&sm.vt[16 * q + r16][32 * s + 16 + 4 * g]);
        const bf16x8 vf = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
        for (int i = 0; i < AP; ++i) o[i][q] = mfma16(as_bf16x8(pf[i][s]), vf, o[i][q]);
      }
  }
  if (!active) return;

  // epilogue: out = g O_s + (1 - g) O_L for rows t = T0 + 16 i + 4 g + r
  const float* gate = a.gate_part;
  const float* olin = a.o_lin;
  bf16_t* out = (bf16_t*)a.out;
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    float lt = lrun[i];
    lt += __shfl_xor(lt, 16, WAVE);
    lt += __shfl_xor(lt, 32, WAVE);
    const float inv = 1.f / lt;  // every causal row selects at least itself
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ir = __shfl(inv, 4 * g + r, WAVE);
      const int t = T0 + 16 * i + 4 * g + r;
      if (t >= n) continue;
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
  const int G = a.sh.H_q / a.sh.H_kv;
  const int npb = (a.n + AQ - 1) / AQ;
  const dim3 grid((unsigned)(npb * a.sh.B * a.sh.H_kv * ((G + 3) / 4)));
  if (a.sh.d == 128) klaunch(k_attn_prefill_mfma<128>, grid, dim3(256), 0, st, a);
  else klaunch(k_attn_prefill_mfma<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
