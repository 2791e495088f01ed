// Launch interface of the prefill kernels.
#pragma once
#include "lisa_common.h"
#include "lisa_kernels.h"

namespace lisa {

constexpr int GMAX_GATE = 64;  // query heads supported by the gate kernels

struct IndexScoreArgs {
  Shape sh;
  int n;                // tokens per sequence
  int row0;             // first query row scored (rows below take every key)
  int stored_rows;      // score rows stored per sequence
  const void* q_idx;    // [B, n, H_I, d_I]
  const void* k_idx;    // [B, cap, H_Ik, d_I]
  const float* w_idx;   // [H_I]
  float* scores;        // row (b, t) at scores + (b*stored_rows + t - row0)*ld
  int64_t ld;
};
hipError_t launch_index_scores(const IndexScoreArgs& a, hipStream_t st);

struct GateArgs {
  Shape sh;
  int n_rows;           // B*n
  const void* x;        // [n_rows, hidden]
  const void* w_gate;   // [hidden, H_q]
  float* gate_part;     // [n_rows, chunks, H_q]
  bf16_t* w_t;          // MFMA path: W_g transposed, [H_q rounded up to 16, hidden]
};
int prefill_gate_chunks(const Shape& sh);
hipError_t launch_gate_logits(const GateArgs& a, hipStream_t st);

struct LinearArgs {
  Shape sh;
  int n;                // tokens per sequence
  const void *q_lin, *k_lin, *v_lin;  // [B, n, H_L, d]
  float* S;             // [B, H_L, d, d] in place
  const float* z_in;    // [B, H_L, d]
  float* z_out;         // [B, H_L, d] (must not alias z_in)
  float* o_lin;         // nullable [B, n, H_L, d]: outputs (normalised unless flagged)
};
hipError_t launch_linear_recurrent(const LinearArgs& a, hipStream_t st);

// Chunked linear branch on bf16 MFMA (head dim 64 or 128).
struct LinearChunkArgs {
  Shape sh;
  int n;                // tokens per sequence
  const void *q_lin, *k_lin, *v_lin;  // [B, n, H_L, d] bf16
  float* S;             // [B, H_L, d, d]: in S_0, out S_n
  float* z;             // [B, H_L, d]:    in z_0, out z_n
  float* seg_state;     // [B, H_L, nseg, d*d + d] segment states (workspace)
  int nseg, seg_len;    // segments of whole 64-token chunks
  int in_place;         // sums kernel only: add the whole sequence to S, z
  float* o_lin;         // [B, n, H_L, d] outputs (normalised unless flagged)
};
bool linear_mfma_supported(const Shape& sh);
void linear_segments(const Shape& sh, int n, int& nseg, int& seg_len);
size_t linear_seg_floats(const Shape& sh, int n);
hipError_t launch_linear_seg_sums(const LinearChunkArgs& a, hipStream_t st);
hipError_t launch_linear_seg_prefix(const LinearChunkArgs& a, hipStream_t st);
hipError_t launch_linear_chunks(const LinearChunkArgs& a, hipStream_t st);
// Masked sparse attention of the prefill on bf16 MFMA (head dim 64 or 128).
struct AttnMaskArgs {
  Shape sh;
  int n;                    // tokens per sequence
  const void* q;            // [B, n, H_q, d]
  const void *k_cache, *v_cache;  // [B, cap, H_kv, d]
  const uint32_t* mask;     // [B * n, mask_ld] selection bitmask rows
  int64_t mask_ld;          // words per row (even)
  float scale_log2e;        // log2(e) / sqrt(d)
  const float* gate_part;   // [B * n, H_q] gate logits
  const float* o_lin;       // [B, n, H_q, d] linear-branch outputs
  void* out;                // [B, n, H_q, d]
  int window;               // sliding window of sh.M positions: no mask rows are read, and key
                            // tiles before every row's window are skipped
  const uint32_t* occ;      // nullable: tile occupancy per 32 query rows ([B, ceil(n/32), occ_ld],
                            // see SelectArgs); a block skips the key tiles its rows never select
  int64_t occ_ld;
};
constexpr int ATTN_MAX_TILES = 1024;  // key tiles of 64 a block can list (n <= 65536)
bool attn_mfma_supported(const Shape& sh);
int64_t attn_mask_ld(int n);
hipError_t launch_attn_prefill_mfma(const AttnMaskArgs& a, hipStream_t st);
// Index lists of the sliding window: row t of each of the B sequences gets
// max(0, t+1-M)..t ascending, then -1 ([B, n, M] int32).
hipError_t launch_window_index(int32_t* idx, int B, int n, int M, hipStream_t st);

// Index scores and gate logits on bf16 MFMA.
bool index_mfma_supported(const Shape& sh);
hipError_t launch_index_scores_mfma(const IndexScoreArgs& a, hipStream_t st);
bool gate_mfma_supported(const Shape& sh);
size_t gate_transpose_elems(const Shape& sh);
hipError_t launch_gate_transpose(const GateArgs& a, hipStream_t st);
hipError_t launch_gate_mfma(const GateArgs& a, hipStream_t st);

hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t st);

}  // namespace lisa
