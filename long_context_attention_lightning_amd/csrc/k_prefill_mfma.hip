// bf16 MFMA prefill kernels for the indexer scores and the gate logits.
//
//  * index scores ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2):
//    s[t, j] = sum_h w_h ReLU(q_I[t,h] . k_I[j, h H_Ik / H_I]) for the
//    stored rows t and every key j <= t.  Per head the dot products are one
//    MFMA contraction over d_I; ReLU and w_h are applied to the fp32 result.
//    Tiles are computed transposed (keys along the accumulator rows) so that
//    each lane holds four consecutive keys of one query row and stores them
//    as one float4.  The streaming form (query rows held in registers, key
//    tiles walked) serves the common head shapes; the per-head tile form
//    is kept for the others.
//  * gate logits (Section 3.3 Eq. 5): x[row] . W_g[:, h] as one GEMM over
//    the hidden dimension; the sigmoid is applied where the gate is used.
#include "lisa_common.h"
#include "lisa_kernels.h"
#include "lisa_mfma.h"
#include "lisa_prefill.h"

namespace lisa {

// ---------------------------------------------------------------------------
// index scores, per-head tile form (head shapes without a streaming
// instantiation): block = 128 query rows x 128 keys, wave = 64 x 64 (4 x 4
// tiles of 16 x 16).  Per indexer head the block stages the head's query and
// key rows in LDS (the next head's rows are loaded into registers meanwhile),
// and every wave reads its MFMA operands from there.
// ---------------------------------------------------------------------------
constexpr int IX_T = 128;          // query rows and keys per block
constexpr int IX_PAD = 8;

template <int DI>
struct IndexShared {
  bf16_t q[IX_T][DI + IX_PAD];
  bf16_t k[IX_T][DI + IX_PAD];
};

template <int DI>
__global__ __launch_bounds__(256) void k_index_scores_mfma(IndexScoreArgs a) {
  __shared__ IndexShared<DI> sm;
  const Shape& sh = a.sh;
  const int b = blockIdx.z;
  const int T0 = IX_T * blockIdx.y, J0 = IX_T * blockIdx.x;
  if (J0 > T0 + IX_T - 1 || T0 + IX_T <= a.row0) return;  // above the diagonal / not stored
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int tw = T0 + 64 * (wave >> 1), jw = J0 + 64 * (wave & 1);
  const bool live = jw <= tw + 63;  // some key of the wave's tiles is causal for some row
  const int R = sh.H_I / sh.H_Ik;
  const bf16_t* qb = (const bf16_t*)a.q_idx + (size_t)b * a.n * sh.H_I * DI;
  const bf16_t* kb = (const bf16_t*)a.k_idx + (size_t)b * sh.cap * sh.H_Ik * DI;

  // staging: the block's 128 rows of one head, DI / 8 vectors of 16 B each
  constexpr int NV = IX_T * DI / 8 / 256;
  uint4 rq[NV], rk[NV];
  auto fetch = [&](int h) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = tid + 256 * m;
      const int row = e / (DI / 8), c8 = e % (DI / 8);
      rq[m] = ld16(qb + ((size_t)min(T0 + row, a.n - 1) * sh.H_I + h) * DI + 8 * c8);
      rk[m] = ld16(kb + ((size_t)min(J0 + row, a.n - 1) * sh.H_Ik + h / R) * DI + 8 * c8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = tid + 256 * m;
      const int row = e / (DI / 8), c8 = e % (DI / 8);
      *reinterpret_cast<uint4*>(&sm.q[row][8 * c8]) = rq[m];
      *reinterpret_cast<uint4*>(&sm.k[row][8 * c8]) = rk[m];
    }
  };

  f32x4 sc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[i][c] = zero4();
  const int qr0 = 64 * (wave >> 1), kr0 = 64 * (wave & 1);  // the wave's rows in the staged tiles
  fetch(0);
  for (int h = 0; h < sh.H_I; ++h) {
    __syncthreads();  // readers of the previous head are done
    stage();
    __syncthreads();
    if (h + 1 < sh.H_I) fetch(h + 1);
    if (!live) continue;
    const float w = a.w_idx[h];
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DI; k0 += 32) {
      bf16x8 qf[4], kf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = as_bf16x8(lds_read16(&sm.q[qr0 + 16 * i + r16][k0 + 8 * g]));
#pragma unroll
      for (int c = 0; c < 4; ++c) kf[c] = as_bf16x8(lds_read16(&sm.k[kr0 + 16 * c + r16][k0 + 8 * g]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = mfma16(kf[c], qf[i], acc[i][c]);  // [key][query]
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[i][c][r] = fmaf(w, fmaxf(acc[i][c][r], 0.f), sc[i][c][r]);
  }
  if (!live) return;
  // lane holds s[t = tw + 16 i + r16][j = jw + 16 c + 4 g + r]; keys past t are written as 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tw + 16 * i + r16;
    if (t < a.row0 || t >= a.n) continue;
    float* orow = a.scores + ((size_t)b * a.stored_rows + (t - a.row0)) * a.ld;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = jw + 16 * c + 4 * g;
      if (j > t) continue;
      float4 v;
      v.x = sc[i][c][0];
      v.y = j + 1 <= t ? sc[i][c][1] : 0.f;
      v.z = j + 2 <= t ? sc[i][c][2] : 0.f;
      v.w = j + 3 <= t ? sc[i][c][3] : 0.f;
      *reinterpret_cast<float4*>(orow + j) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// index scores, streaming form: a block holds 256 query rows (8 waves x 32)
// with all their indexer heads in registers and walks a run of up to
// IS_KC 64-key tiles of their causal prefix.  Each key tile (every key head)
// is loaded once per block into registers while the previous tile is
// computed, staged in one of two LDS buffers, and its scores are stored as
// soon as they are summed, so loads, MFMAs and the score stores of
// consecutive tiles overlap.  Keys past a row are written as 0 inside the
// float4 that holds the row's last key; later float4 groups are not written.
// ---------------------------------------------------------------------------
constexpr int IS_THREADS = 512;
constexpr int IS_Q = IS_THREADS / WAVE * 32;  // query rows per block
constexpr int IS_K = 64;   // keys per tile
constexpr int IS_KC = 7;   // key tiles per block (5-7 measured fastest at 16K tokens; 4 and 8 about 25% slower)

template <int DI, int HI, int HK>
__global__ __launch_bounds__(IS_THREADS) void k_index_scores_stream(IndexScoreArgs a, int qt0) {
  constexpr int KS = DI / 32;          // MFMA k-steps per head
  constexpr int EK = HK * DI;          // key row (every key head)
  constexpr int LDK = EK + 16;         // LDS row stride: 8 dwords mod 64 when EK is a multiple of 128
  constexpr int NVT = IS_K * EK / 8;  // 16-byte vectors of a key tile
  constexpr int NV = (NVT + IS_THREADS - 1) / IS_THREADS;  // per thread
  static_assert(NVT % IS_THREADS == 0 || NVT < IS_THREADS, "key tile split");
  __shared__ bf16_t ks[2][IS_K][LDK];
  const Shape& sh = a.sh;
  const int b = blockIdx.z;
  const int t0 = IS_Q * (qt0 + (int)blockIdx.y);
  const int nkt = (min(t0 + IS_Q, a.n) + IS_K - 1) / IS_K;  // key tiles of the block's prefix
  const int kt0 = IS_KC * (int)blockIdx.x;
  if (kt0 >= nkt) return;
  const int kt1 = min(nkt, kt0 + IS_KC);
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const bf16_t* qb = (const bf16_t*)a.q_idx + (size_t)b * a.n * HI * DI;
  const bf16_t* kb = (const bf16_t*)a.k_idx + (size_t)b * sh.cap * EK;

  // the wave's 32 query rows, every head: B operands of the score MFMAs
  uint4 qv[2][HI][KS];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = min(t0 + 32 * wave + 16 * i + r16, a.n - 1);
#pragma unroll
    for (int h = 0; h < HI; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[i][h][s] = ld16(qb + ((size_t)t * HI + h) * DI + 32 * s + 8 * g);
  }
  float wv[HI];
#pragma unroll
  for (int h = 0; h < HI; ++h) wv[h] = a.w_idx[h];

  // the sequence's key rows through a buffer resource limited to its n rows:
  // loads past them return zeros (those keys are never stored)
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, (int)((size_t)a.n * EK * 2), 0x00020000);
  const uint32_t koff = (uint32_t)(((tid / (EK / 8)) * EK + 8 * (tid % (EK / 8))) * 2);
  uint4 kr[NV];
  auto fetch = [&](int kt) {  // vector m of the thread is IS_THREADS m vectors further
    const uint32_t off = koff + (uint32_t)kt * (IS_K * EK * 2);
#pragma unroll
    for (int m = 0; m < NV; ++m)
      if (NVT >= IS_THREADS || tid < NVT)
        kr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kres, off + 16u * IS_THREADS * m, 0, 0));
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = tid + IS_THREADS * m;
      const int row = e / (EK / 8), c8 = e % (EK / 8);
      if (e < NVT) *reinterpret_cast<uint4*>(&ks[buf][row][8 * c8]) = kr[m];
    }
  };

  fetch(kt0);
  stage(0);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    if (kt + 1 < kt1) fetch(kt + 1);
    f32x4 sc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[i][c] = zero4();
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      const int kc = (h / (HI / HK)) * DI;  // the head's key columns
      f32x4 acc[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = as_bf16x8(lds_read16(&ks[buf][16 * c + r16][kc + 32 * s + 8 * g]));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[i][c] = mfma16(kf[c], as_bf16x8(qv[i][h][s]), acc[i][c]);  // [key][query]
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[i][c][r] = fmaf(wv[h], fmaxf(acc[i][c][r], 0.f), sc[i][c][r]);
    }
    // lane holds s[t = t0 + 32 wave + 16 i + r16][j = 64 kt + 16 c + 4 g + r]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = t0 + 32 * wave + 16 * i + r16;
      if (t < a.row0 || t >= a.n) continue;
      float* orow = a.scores + ((size_t)b * a.stored_rows + (t - a.row0)) * a.ld;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = IS_K * kt + 16 * c + 4 * g;
        if (j > t) continue;
        float4 v;
        v.x = sc[i][c][0];
        v.y = j + 1 <= t ? sc[i][c][1] : 0.f;
        v.z = j + 2 <= t ? sc[i][c][2] : 0.f;
        v.w = j + 3 <= t ? sc[i][c][3] : 0.f;
        *reinterpret_cast<float4*>(orow + j) = v;
      }
    }
    if (kt + 1 < kt1) stage(buf ^ 1);  // the buffer every wave finished reading before the last barrier
    __syncthreads();
  }
}

template <int DI, int HI>
static bool launch_is_hk(const IndexScoreArgs& a, dim3 grid, int qt0, hipStream_t st) {
  if (a.sh.H_Ik == HI) klaunch((k_index_scores_stream<DI, HI, HI>), grid, dim3(IS_THREADS), 0, st, a, qt0);
  else if (a.sh.H_Ik == 1) klaunch((k_index_scores_stream<DI, HI, 1>), grid, dim3(IS_THREADS), 0, st, a, qt0);
  else return false;
  return true;
}

template <int DI>
static bool launch_is_di(const IndexScoreArgs& a, dim3 grid, int qt0, hipStream_t st) {
  switch (a.sh.H_I) {
    case 1: return launch_is_hk<DI, 1>(a, grid, qt0, st);
    case 2: return launch_is_hk<DI, 2>(a, grid, qt0, st);
    case 4: if constexpr (DI <= 64) return launch_is_hk<DI, 4>(a, grid, qt0, st); else return false;
    default: return false;
  }
}

// The streaming form when the shape has one of its instantiations; false
// (nothing launched) otherwise.
static bool launch_index_scores_stream(const IndexScoreArgs& a, hipStream_t st) {
  if ((size_t)a.n * a.sh.H_Ik * a.sh.d_I * 2 > 0x7fffffffu) return false;  // 31-bit buffer offsets
  const int qt0 = a.row0 / IS_Q;
  const int nqt = (a.n + IS_Q - 1) / IS_Q - qt0;
  const int nkt = (a.n + IS_K - 1) / IS_K;
  const dim3 grid((unsigned)((nkt + IS_KC - 1) / IS_KC), (unsigned)nqt, (unsigned)a.sh.B);
  switch (a.sh.d_I) {
    case 32: return launch_is_di<32>(a, grid, qt0, st);
    case 64: return launch_is_di<64>(a, grid, qt0, st);
    case 128: return launch_is_di<128>(a, grid, qt0, st);
    default: return false;
  }
}

bool index_mfma_supported(const Shape& sh) { return sh.dtype == 1 && (sh.d_I == 32 || sh.d_I == 64 || sh.d_I == 128); }

hipError_t launch_index_scores_mfma(const IndexScoreArgs& a, hipStream_t st) {
  if (a.n - a.row0 <= 0) return hipSuccess;
  if (launch_index_scores_stream(a, st)) return hipGetLastError();
  const dim3 grid((unsigned)((a.n + IX_T - 1) / IX_T), (unsigned)((a.n + IX_T - 1) / IX_T), (unsigned)a.sh.B);
  switch (a.sh.d_I) {
    case 32: klaunch(k_index_scores_mfma<32>, grid, dim3(256), 0, st, a); break;
    case 64: klaunch(k_index_scores_mfma<64>, grid, dim3(256), 0, st, a); break;
    default: klaunch(k_index_scores_mfma<128>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gate logits: W_g [hidden, H_q] is first transposed into [H_pad, hidden]
// (H_pad = H_q rounded up to 16, zero rows) so that both MFMA operands are
// 16-byte row reads; block = 16 rows x H_pad heads (below).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gate_transpose(GateArgs a) {
  const Shape& sh = a.sh;
  const int hp = (sh.H_q + 15) / 16 * 16;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)hp * sh.hidden) return;
  const int h = (int)(e / sh.hidden), c = (int)(e % sh.hidden);
  a.w_t[e] = h < sh.H_q ? ((const bf16_t*)a.w_gate)[(size_t)c * sh.H_q + h] : (bf16_t)0;
}

// Block = 16 rows; its four waves split the hidden dimension (wave w takes
// the w-th quarter of the 32-wide contraction steps) so that four waves per
// SIMD keep loads in flight, and their partial logits are summed in LDS.
template <int NH>  // head tiles of 16
__global__ __launch_bounds__(256) void k_gate_mfma(GateArgs a) {
  __shared__ float red[4][16][16 * NH + 1];
  const Shape& sh = a.sh;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = min(row0 + r16, a.n_rows - 1);
  const bf16_t* x = (const bf16_t*)a.x + (size_t)row * sh.hidden + 8 * g;
  const bf16_t* w = a.w_t + (size_t)r16 * sh.hidden + 8 * g;
  const int steps = sh.hidden / 32;
  const int s0 = steps * wave / 4, s1 = steps * (wave + 1) / 4;
  f32x4 acc[NH];
#pragma unroll
  for (int q = 0; q < NH; ++q) acc[q] = zero4();
  int st = s0;
  for (; st + 4 <= s1; st += 4) {  // four contraction steps per iteration, loads first
    uint4 xv[4], wv[4][NH];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 32 * (st + u);
      xv[u] = ld16(x + c);
#pragma unroll
      for (int q = 0; q < NH; ++q) wv[u][q] = ld16(w + (size_t)16 * q * sh.hidden + c);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < NH; ++q) acc[q] = mfma16(as_bf16x8(wv[u][q]), as_bf16x8(xv[u]), acc[q]);
  }
  for (; st < s1; ++st) {
    const int c = 32 * st;
    const uint4 xv = ld16(x + c);
#pragma unroll
    for (int q = 0; q < NH; ++q)
      acc[q] = mfma16(as_bf16x8(ld16(w + (size_t)16 * q * sh.hidden + c)), as_bf16x8(xv), acc[q]);
  }
  // lane holds the partial logit[row0 + r16][h = 16 q + 4 g + r]
#pragma unroll
  for (int q = 0; q < NH; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r16][16 * q + 4 * g + r] = acc[q][r];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * sh.H_q; e += 256) {
    const int rr = e / sh.H_q, h = e % sh.H_q;
    if (row0 + rr < a.n_rows)
      a.gate_part[(size_t)(row0 + rr) * sh.H_q + h] = red[0][rr][h] + red[1][rr][h] + red[2][rr][h] + red[3][rr][h];
  }
}

bool gate_mfma_supported(const Shape& sh) { return sh.dtype == 1 && sh.hidden % 32 == 0 && sh.H_q <= 64; }

size_t gate_transpose_elems(const Shape& sh) { return (size_t)((sh.H_q + 15) / 16 * 16) * sh.hidden; }

hipError_t launch_gate_transpose(const GateArgs& a, hipStream_t st) {
  const size_t te = gate_transpose_elems(a.sh);
  klaunch(k_gate_transpose, dim3((unsigned)((te + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gate_mfma(const GateArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_rows + 15) / 16));
  switch ((a.sh.H_q + 15) / 16) {
    case 1: klaunch(k_gate_mfma<1>, grid, dim3(256), 0, st, a); break;
    case 2: klaunch(k_gate_mfma<2>, grid, dim3(256), 0, st, a); break;
    case 3: klaunch(k_gate_mfma<3>, grid, dim3(256), 0, st, a); break;
    default: klaunch(k_gate_mfma<4>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace lisa
