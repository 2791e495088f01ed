// Indexer candidate dropout ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2:
// early in training the top 1.2 M candidates are taken, a random 20% of them
// is masked out, and the sparse attention is filled from the rest, the ratio
// being lowered as training goes on).  Per score row:
//   1. the top n_cand positions (the library's select, as a bitmask);
//   2. k_dropout_compact: the survivors (candidates whose caller-drawn
//      uniform u is at least p), in position order, as a short row of their
//      scores and positions, with its length;
//   3. the top-M select of each short row (ties go to the later entry, which
//      is the later position);
//   4. k_dropout_gather: the selected entries' positions, ascending, -1 padded.
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

__device__ __forceinline__ int dropout_row_len(const DropoutArgs& a, int r) {
  return a.prefill ? r % a.rows_per_seq + 1 : a.seq_lens[r];
}

// One block per row, in rounds of 1024 positions: thread t takes positions
// 1024 i + 4 t .. + 3, so every wave reads 256 consecutive uniforms and
// scores (two 16-byte vectors per lane, issued with the mask word before any
// of them is used).  A block scan of the survivor counts of the round, added
// to the survivors of the earlier rounds, gives each thread its output
// offset, so the survivors come out in position order and each wave's writes
// fill one consecutive range.  One barrier per round: the scan's wave totals
// alternate between two slots.
__global__ __launch_bounds__(256) void k_dropout_compact(DropoutArgs a) {
  __shared__ uint32_t wsum[2][4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int len = dropout_row_len(a, r);
  const uint32_t* mrow = a.mask + (size_t)r * a.mask_ld;
  const float* urow = a.u + (size_t)r * a.ld;
  const float* srow = a.scores + (size_t)r * a.ld;
  float* cs = a.cscore + (size_t)r * a.cld;
  int32_t* cp = a.cpos + (size_t)r * a.cld;
  uint32_t base = 0;  // survivors of the earlier rounds
  const int rounds = (len + 1023) / 1024;
  for (int i = 0; i < rounds; ++i) {
    const int p = 1024 * i + 4 * tid;  // 4-aligned; p < len implies p + 3 < ld
    uint32_t m4 = 0;
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f), sc = u;
    if (p < len) {
      m4 = (mrow[p >> 5] >> (p & 31)) & 0xfu;
      u = *reinterpret_cast<const float4*>(urow + p);
      sc = *reinterpret_cast<const float4*>(srow + p);
      if (len - p < 4) m4 &= (1u << (len - p)) - 1u;  // positions past the row
    }
    const uint32_t keep = ((m4 & 1u) && u.x >= a.p ? 1u : 0u) | ((m4 & 2u) && u.y >= a.p ? 2u : 0u) |
                          ((m4 & 4u) && u.z >= a.p ? 4u : 0u) | ((m4 & 8u) && u.w >= a.p ? 8u : 0u);
    const uint32_t c = (uint32_t)__builtin_popcount(keep);
    const uint32_t incl = wave_incl_scan_u32(c);
    if (lane == WAVE - 1) wsum[i & 1][wave] = incl;
    __syncthreads();
    uint32_t o = base + incl - c, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = wsum[i & 1][w];
      if (w < wave) o += t;
      tot += t;
    }
    base += tot;
    if (keep & 1u) { cs[o] = sc.x; cp[o] = p; ++o; }
    if (keep & 2u) { cs[o] = sc.y; cp[o] = p + 1; ++o; }
    if (keep & 4u) { cs[o] = sc.z; cp[o] = p + 2; ++o; }
    if (keep & 8u) { cs[o] = sc.w; cp[o] = p + 3; }
  }
  if (tid == 0) a.cnt[r] = (int32_t)base;
}

__global__ __launch_bounds__(256) void k_dropout_gather(DropoutArgs a) {
  const int r = blockIdx.x;
  const int32_t* __restrict__ in = a.idx2 + (size_t)r * a.M;
  const int32_t* __restrict__ cp = a.cpos + (size_t)r * a.cld;
  int32_t* __restrict__ out = a.idx_out + (size_t)r * a.M;
  constexpr int U = 8;  // entries per thread in flight
  for (int k0 = threadIdx.x; k0 < a.M; k0 += 256 * U) {
    int e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) e[u] = k0 + 256 * u < a.M ? in[k0 + 256 * u] : -1;
    int p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] = e[u] >= 0 ? cp[e[u]] : -1;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + 256 * u < a.M) out[k0 + 256 * u] = p[u];
  }
}

hipError_t launch_dropout_compact(const DropoutArgs& a, hipStream_t st) {
  klaunch(k_dropout_compact, dim3((unsigned)a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dropout_gather(const DropoutArgs& a, hipStream_t st) {
  klaunch(k_dropout_gather, dim3((unsigned)a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
