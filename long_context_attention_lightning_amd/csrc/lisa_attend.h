// Gathered GQA attention of one split of selected cache rows, shared by the
// decode attention kernels ("LISA", arXiv 2607.19358v1, Section 3.2: softmax
// attention over the M selected positions).
#pragma once
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"

namespace lisa {

// ---------------------------------------------------------------------------
// gathered GQA attention
// ---------------------------------------------------------------------------
// Block = (row, KV head, split).  A "slot" of D/VEC lanes owns one gathered
// row of K (then V) at a time; each slot keeps its own online-softmax state
// (max, sum, accumulator) for the GT query heads of the group and loads the
// K and V rows of AT_RP positions at once, so one round costs two dependent
// memory trips (the index, then the rows).  Slots are merged with xor
// shuffles inside the wave and through LDS across the four waves.
constexpr int AT_THREADS = 256;
constexpr int AT_RP = 4;        // positions per slot per round
constexpr int AT_MAX_SPLITS = 32;


__device__ __forceinline__ float scale_from(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : exp2f(m_old - m_new);
}

template <int NW, int GT, int D>
struct AttnMergeShared {
  float wm[NW][GT], wl[NW][GT];
  float wacc[NW][GT * D];
};

// Merge the NWM per-wave (max, sum, accumulator) entries of one split and
// write the split partial, or the gated output when there is one split.
template <typename T, int D, int GT, int NWM, int THREADS, int NWS>
__device__ __forceinline__ void attend_epilogue(const AttnArgs& a, int r, int g, int s,
                                                const AttnMergeShared<NWS, GT, D>& ms) {
  const Shape& sh = a.sh;
  const int G = sh.H_q / sh.H_kv;
  const int tid = threadIdx.x;
  const int GD = G * D;
  const int PS = GD + 2 * G;
  float* mypart = a.nsplit > 1 ? a.part + (((size_t)r * sh.H_kv + g) * a.nsplit + s) * PS : nullptr;
  for (int e = tid; e < GD; e += THREADS) {
    const int hh = e / D, dim = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWM; ++w) mx = fmaxf(mx, ms.wm[w][hh]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NWM; ++w) {
      const float f = scale_from(ms.wm[w][hh], mx);
      l = fmaf(ms.wl[w][hh], f, l);
      o = fmaf(ms.wacc[w][e], f, o);
    }
    if (mypart) {
      // split partial: unnormalised accumulator, max and sum; the combine
      // kernel merges the splits (the kernel boundary orders the writes
      // before its reads, with no device-scope fence here)
      mypart[e] = o;
      if (dim == 0) {
        mypart[GD + hh] = mx;
        mypart[GD + G + hh] = l;
      }
      continue;
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

// Attention of query row r and KV head g over the selected entries
// [i0, i1) of split s (pos_of(i) gives the cache position of entry i), by
// a block of THREADS threads; writes the split partial, or the gated
// output when there is one split.
template <typename T, int D, int GT, int THREADS, int RP, typename PosFn>
__device__ __forceinline__ void attend_split(const AttnArgs& a, int r, int g, int s, int len, int i0, int i1,
                                             PosFn pos_of, AttnMergeShared<THREADS / WAVE, GT, D>& ms) {
  using V = Vec<T>;
  constexpr int VEC = V::N;
  constexpr int LG = D / VEC;            // lanes per row of one head
  constexpr int NG = THREADS / LG;       // slots
  constexpr int NW = THREADS / WAVE;
  constexpr int ROUND = NG * RP;         // positions per round
  const Shape& sh = a.sh;
  const int G = sh.H_q / sh.H_kv;
  const int b = r / a.rows_per_seq;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int ps = tid / LG, li = tid % LG;
  const float scale = 1.4426950408889634f * rsqrtf((float)D);

  float q[GT][VEC];
  const T* qrow = (const T*)a.q + ((size_t)r * sh.H_q + (size_t)g * G) * D + li * VEC;
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    V::unpack(ld16(qrow + (size_t)min(hh, G - 1) * D), q[hh]);
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[hh][v] *= scale;
  }
  float mrun[GT], lrun[GT], acc[GT][VEC];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[hh][v] = 0.f;
  }
  const size_t row_stride = (size_t)sh.H_kv * D;
  const T* kb = (const T*)a.k_cache + ((size_t)b * sh.cap * sh.H_kv + g) * D + li * VEC;
  const T* vb = (const T*)a.v_cache + ((size_t)b * sh.cap * sh.H_kv + g) * D + li * VEC;

  for (int c0 = i0; c0 < i1; c0 += ROUND) {
    int pos[RP];
    bool valid[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int i = c0 + ps + NG * k;
      valid[k] = i < i1;
      const int ii = min(i, i1 - 1);
      const int pp = pos_of(ii);
      pos[k] = min(max(pp, 0), len - 1);  // defensive: never read outside the row
    }
    uint4 kr[RP], vr[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      kr[k] = ld16(kb + (size_t)pos[k] * row_stride);
      vr[k] = ld16(vb + (size_t)pos[k] * row_stride);
    }
    float lg[RP][GT];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      float kf[VEC];
      V::unpack(kr[k], kf);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = fmaf(q[hh][v], kf[v], dot);
        lg[k][hh] = group_sum(dot, LG);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float mx = mrun[hh];
#pragma unroll
      for (int k = 0; k < RP; ++k)
        if (valid[k]) mx = fmaxf(mx, lg[k][hh]);
      const float f = scale_from(mrun[hh], mx);
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < RP; ++k) {
        const float p = valid[k] ? exp2f(lg[k][hh] - mx) : 0.f;
        lg[k][hh] = p;
        psum += p;
      }
      lrun[hh] = lrun[hh] * f + psum;
      mrun[hh] = mx;
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[hh][v] *= f;
    }
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      float vf[VEC];
      V::unpack(vr[k], vf);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[hh][v] = fmaf(lg[k][hh], vf[v], acc[hh][v]);
    }
  }

  // merge the slots of the wave (xor partners hold the same dimensions)
#pragma unroll
  for (int off = LG; off < WAVE; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float mo = __shfl_xor(mrun[hh], off, WAVE);
      const float lo = __shfl_xor(lrun[hh], off, WAVE);
      const float mn = fmaxf(mrun[hh], mo);
      const float f1 = scale_from(mrun[hh], mn), f2 = scale_from(mo, mn);
      lrun[hh] = lrun[hh] * f1 + lo * f2;
      mrun[hh] = mn;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float ao = __shfl_xor(acc[hh][v], off, WAVE);
        acc[hh][v] = acc[hh][v] * f1 + ao * f2;
      }
    }
  }
  if (lane < LG) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      if (lane == 0) {
        ms.wm[wave][hh] = mrun[hh];
        ms.wl[wave][hh] = lrun[hh];
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) ms.wacc[wave][hh * D + li * VEC + v] = acc[hh][v];
    }
  }
  __syncthreads();

  attend_epilogue<T, D, GT, NW, THREADS>(a, r, g, s, ms);
}

// ---------------------------------------------------------------------------
// The same split on bf16 MFMA.  The block's first NWA waves take 32 entries
// each of every (32 NWA)-entry chunk of the split: S^T = K Q^T (gathered K
// rows as the A operand, the G query heads of the KV group as the 16 columns,
// rows past G zero), online softmax per head along the accumulator rows, then
// O = P V with P taken from the accumulators (contraction order permuted
// alike in P and in V) and V transposed through LDS as packed position pairs.
// Each attending wave keeps its own online-softmax state and the epilogue
// merges them; waves past NWA (the fused select kernel has eight waves, two
// of which attend) only join the block's barriers.
// ---------------------------------------------------------------------------
template <int D, int GT, int NWA>
struct AttnMfmaShared {
  union {  // the merge state is written once no wave reads its V tile any more
    bf16_t vt[NWA][D][32 + 8];
    AttnMergeShared<NWA, GT, D> ms;
  };
};

template <int D, int GT, int THREADS, int NWA, typename PosFn>
__device__ __forceinline__ void attend_split_mfma(const AttnArgs& a, int r, int g, int s, int len, int i0, int i1,
                                                  PosFn pos_of, AttnMfmaShared<D, GT, NWA>& sm) {
  static_assert(GT <= 8, "query heads per KV head");
  const Shape& sh = a.sh;
  const int G = sh.H_q / sh.H_kv;
  const int b = r / a.rows_per_seq;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g4 = lane >> 4;
  const float scale = 1.4426950408889634f * rsqrtf((float)D);
  float mrun = -INFINITY, lrun = 0.f;  // of query head r16
  f32x4 o[D / 16];
#pragma unroll
  for (int q = 0; q < D / 16; ++q) o[q] = zero4();
  if (wave < NWA) {
    const size_t row_stride = (size_t)sh.H_kv * D;
    const bf16_t* kb = (const bf16_t*)a.k_cache + (size_t)b * sh.cap * row_stride + (size_t)g * D;
    const bf16_t* vb = (const bf16_t*)a.v_cache + (size_t)b * sh.cap * row_stride + (size_t)g * D;
    // Q^T operand: column r16 = query head of the group (zero past G)
    bf16x8 qf[D / 32];
    {
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)r * sh.H_q + (size_t)g * G + min(r16, G - 1)) * D;
#pragma unroll
      for (int k = 0; k < D / 32; ++k) {
        const uint4 v = ld16(qrow + 32 * k + 8 * g4);
        qf[k] = as_bf16x8(r16 < G ? v : make_uint4(0u, 0u, 0u, 0u));
      }
    }
    bf16_t(*vt)[32 + 8] = sm.vt[wave];
    for (int c0 = i0 + 32 * wave; c0 < i1; c0 += 32 * NWA) {
      // gathered rows: K of entries c0 + 16 c + r16; V of entry pairs c0 + 2 r16 + u
      int pk[2], pv[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) pk[c] = min(max(pos_of(min(c0 + 16 * c + r16, i1 - 1)), 0), len - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) pv[u] = min(max(pos_of(min(c0 + 2 * r16 + u, i1 - 1)), 0), len - 1);
      bf16x8 kf[2][D / 32];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < D / 32; ++k) kf[c][k] = as_bf16x8(ld16(kb + (size_t)pk[c] * row_stride + 32 * k + 8 * g4));
      uint4 vr[D / 32][2];
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
#pragma unroll
        for (int u = 0; u < 2; ++u) vr[m][u] = ld16(vb + (size_t)pv[u] * row_stride + 8 * (g4 + 4 * m));
      // scores: lane holds s[entry c0 + 16 c + 4 g4 + rr][head r16]
      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x4 st = zero4();
#pragma unroll
        for (int k = 0; k < D / 32; ++k) st = mfma16(kf[c][k], qf[k], st);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool on = c0 + 16 * c + 4 * g4 + rr < i1;
          sv[c][rr] = on ? st[rr] * scale : -INFINITY;
          mx = fmaxf(mx, sv[c][rr]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float mnew = fmaxf(mrun, mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(mrun - muse);
      mrun = mnew;
      uint32_t pb[2][4];
      float ls = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pb[c][rr] = f2bf(exp2f(sv[c][rr] - muse));
          ls += bf2f(pb[c][rr]);
        }
      lrun = lrun * alpha + ls;
      const bf16x8 pf = as_bf16x8(make_uint4(pb[0][0] | (pb[0][1] << 16), pb[0][2] | (pb[0][3] << 16),
                                             pb[1][0] | (pb[1][1] << 16), pb[1][2] | (pb[1][3] << 16)));
      // V transposed into LDS: vt[dim][entry pair] as one dword per pair
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const int c8 = g4 + 4 * m;
        const uint32_t x[4] = {vr[m][0].x, vr[m][0].y, vr[m][0].z, vr[m][0].w};
        const uint32_t y[4] = {vr[m][1].x, vr[m][1].y, vr[m][1].z, vr[m][1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint32_t*>(&vt[8 * c8 + 2 * e][2 * r16]) = (x[e] & 0xffffu) | (y[e] << 16);
          *reinterpret_cast<uint32_t*>(&vt[8 * c8 + 2 * e + 1][2 * r16]) = (x[e] >> 16) | (y[e] & 0xffff0000u);
        }
      }
      // O rows are heads 4 g4 + rr: rescale by the alpha of their head
      float ar[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ar[rr] = __shfl(alpha, 4 * g4 + rr, WAVE);
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(&vt[16 * q + r16][4 * g4]);
        const uint2 x1 = *reinterpret_cast<const uint2*>(&vt[16 * q + r16][16 + 4 * g4]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[q][rr] *= ar[rr];
        o[q] = mfma16(pf, as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), o[q]);
      }
    }
    lrun += __shfl_xor(lrun, 16, WAVE);
    lrun += __shfl_xor(lrun, 32, WAVE);
  }
  __syncthreads();  // every wave is done with its V tile
  if (wave < NWA) {
    if (g4 == 0 && r16 < GT) {
      sm.ms.wm[wave][r16] = mrun;
      sm.ms.wl[wave][r16] = lrun;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hh = 4 * g4 + rr;
      if (hh < GT) {
#pragma unroll
        for (int q = 0; q < D / 16; ++q) sm.ms.wacc[wave][hh * D + 16 * q + r16] = o[q][rr];
      }
    }
  }
  __syncthreads();
  attend_epilogue<bf16_t, D, GT, NWA, THREADS>(a, r, g, s, sm.ms);
}

}  // namespace lisa
