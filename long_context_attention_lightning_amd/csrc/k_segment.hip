// Segment state correction of the linear branch ("LISA", arXiv 2607.19358v1,
// Section 3.3 "Segment State Update", Eqs. 6-9): at the end of segment t the
// state change over the segment (Eq. 6) is blended with the mean change of
// the earlier segments (Eqs. 7-8) and the state restarts from the segment's
// start plus that blend (Eq. 9).  The normaliser z is corrected like S.
//
// One elementwise pass over S and z (HBM-bound: 12 bytes read and 12
// written per element), four elements per thread.
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

__global__ __launch_bounds__(256) void k_segment_correct(SegmentArgs a) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // float4 index over S then z
  const size_t nS4 = a.n_S / 4, nz4 = a.n_z / 4;
  float4 *cur, *start, *mean;
  size_t j;
  if (i4 < nS4) {
    cur = reinterpret_cast<float4*>(a.S); start = reinterpret_cast<float4*>(a.S_start);
    mean = reinterpret_cast<float4*>(a.mean_S); j = i4;
  } else if (i4 < nS4 + nz4) {
    cur = reinterpret_cast<float4*>(a.z); start = reinterpret_cast<float4*>(a.z_start);
    mean = reinterpret_cast<float4*>(a.mean_z); j = i4 - nS4;
  } else {
    return;
  }
  const float4 c = cur[j], s = start[j];
  const float4 m = a.t > 1 ? mean[j] : make_float4(0.f, 0.f, 0.f, 0.f);  // no earlier segment: zero
  const float al = a.alpha, bl = 1.f - a.alpha, inv_t = 1.f / (float)a.t;
  float4 o, mn;
  const float* cv = &c.x;
  const float* sv = &s.x;
  const float* mv = &m.x;
  float* ov = &o.x;
  float* nv = &mn.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float grad = cv[e] - sv[e];                      // Eq. 6
    ov[e] = sv[e] + fmaf(bl, grad, al * mv[e]);            // Eqs. 8-9
    nv[e] = fmaf(grad - mv[e], inv_t, mv[e]);              // Eq. 7: mean over segments 1..t
  }
  cur[j] = o;
  start[j] = o;  // the next segment starts from the corrected state
  mean[j] = mn;
}

hipError_t launch_segment_correct(const SegmentArgs& a, hipStream_t st) {
  const size_t n4 = (a.n_S + a.n_z) / 4;
  if (n4 == 0) return hipSuccess;
  klaunch(k_segment_correct, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lisa
