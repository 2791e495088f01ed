// Launch interface of the prefill kernels.
#pragma once
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
hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t st);

}  // namespace lisa
