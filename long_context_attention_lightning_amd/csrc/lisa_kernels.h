// Launch interface between the C-ABI host layer and the HIP kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

struct Shape {
  int B, H_q, H_kv, d, H_I, H_Ik, d_I, H_L, hidden, M, cap, max_len, chunk, dtype;
  unsigned flags;
};

// Start/stop events for the next kernel launch of this host thread. When set,
// the launch goes through hipExtLaunchKernel, which timestamps the kernel's
// own dispatch (the same interval a kernel trace reports).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& next_launch_events();

template <typename F, typename... Args>
inline void klaunch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, Args... args) {
  LaunchEvents& ev = next_launch_events();
  if (ev.start) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev.start, ev.stop, 0, args...);
    ev = LaunchEvents();
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
}

enum KernelId {
  KID_DECODE_PHASE_A = 0,
  KID_SELECT = 1,
  KID_ATTN = 2,
  KID_PREFILL_INDEX = 3,
  KID_PREFILL_GATE = 4,
  KID_PREFILL_LINEAR = 5,
  KID_PREFILL_ATTN = 6,
  KID_LINEAR_UPDATE = 7,
  KID_ATTN_COMBINE = 8,
  KID_PREFILL_LIN_SUMS = 9,
  KID_PREFILL_LIN_PREFIX = 10,
  KID_PREFILL_GATE_PREP = 11,
  KID_SELECT_ATTN = 12,
  KID_SEGMENT = 13,
  KID_MASS_LOGITS = 14,
  KID_MASS_SELECT = 15,
  KID_MASS_REDUCE = 16,
  KID_INDEXER_KL = 17,
  KID_DROPOUT = 18,
  KID_PREFILL_OCCUPANCY = 19,
  KID_COUNT = 20
};

// ---------------------------------------------------------------------------
// decode phase A: indexer scan + cache append + linear state + gate partials
// ---------------------------------------------------------------------------
struct PhaseAArgs {
  Shape sh;
  const int32_t* seq_lens;
  const void *q_idx, *k_idx_new, *k_new, *v_new;
  const void *q_lin, *k_lin, *v_lin, *x, *w_gate;
  const float* w_idx;
  void *k_cache, *v_cache, *k_idx_cache;
  float *S, *z;
  float* scores;       // [B, scores_ld]
  int64_t scores_ld;
  float* o_lin;        // [B, H_L, d] numerators phi(q) S_new
  float* lin_den;      // [B, H_L] denominators phi(q) . z_new (normalised mode)
  float* gate_part;    // [B, gate_chunks, H_q]  (pre-sigmoid partial dots)
  int gate_chunks;
  int append;          // write the new token into the caches
  int do_scores, do_linear, do_gate;
  int linear_output;   // write o_lin
  int32_t* window_idx; // nullable [B, M]: without scoring, the M most recent positions (sliding window)
  int M;
};
hipError_t launch_decode_phase_a(const PhaseAArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// top-M selection of score rows
// ---------------------------------------------------------------------------
struct SelectArgs {
  int n_rows;               // rows to process (decode: B; prefill: B*n)
  int rows_per_seq;         // decode: 1; prefill: n
  int prefill;              // row t of a sequence has length t+1
  const int32_t* seq_lens;  // decode lengths
  const float* scores;      // row (b, t) at scores + (b*stored_rows + t - first_row)*ld
  int64_t ld;
  int first_row;            // first stored score row per sequence (prefill)
  int stored_rows;          // stored score rows per sequence (prefill)
  int M;
  int max_len;              // longest row
  int32_t* idx;             // nullable [n_rows, idx_ld]
  int64_t idx_ld;
  uint32_t* mask;           // nullable [n_rows, mask_ld] selection bitmask
  int64_t mask_ld;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
// Key-tile occupancy of a prefill bitmask ([B, n, mask_ld] words): one row of
// occ_ld words per 32 query rows ([B, ceil(n/32), occ_ld]); bit k of word w
// is set when some row of the group selects a key of key tile 32 w + k (64
// keys per tile).
hipError_t launch_mask_occupancy(const uint32_t* mask, int64_t mask_ld, int B, int n, uint32_t* occ, int64_t occ_ld,
                                 hipStream_t st);

// ---------------------------------------------------------------------------
// gathered GQA softmax attention over selected rows, split + combine + gate
// ---------------------------------------------------------------------------
struct AttnArgs {
  Shape sh;
  int n_rows;               // query rows (decode: B; prefill: B*n)
  int rows_per_seq;         // decode: 1; prefill: n
  int prefill;              // row length t+1 instead of seq_lens[b]
  int dense;                // positions 0..len-1, no idx
  const int32_t* seq_lens;
  const void* q;            // [n_rows, H_q, d]
  const void *k_cache, *v_cache;
  const int32_t* idx;       // [n_rows, idx_ld]
  int64_t idx_ld;
  int nsplit, split_len;    // positions per split
  float* part;              // partials
  const float* gate_part;   // nullable [n_rows, gate_chunks, H_q] pre-sigmoid
  int gate_chunks;
  const float* o_lin;       // [n_rows, H_q, d] (with gate)
  const float* lin_den;     // nullable [n_rows, H_q]: o_lin is divided by it
  void* out;                // [n_rows, H_q, d] T
  int window;               // positions len-m .. len-1 (sliding window) instead of idx
};
// ---------------------------------------------------------------------------
// segment state correction (elementwise over S and z)
// ---------------------------------------------------------------------------
struct SegmentArgs {
  float *S, *z;              // in: state at the segment's end; out: corrected
  float *S_start, *z_start;  // in: state at the segment's start; out: the corrected state
  float *mean_S, *mean_z;    // in: mean direction of segments 1..t-1; out: of 1..t
  size_t n_S, n_z;           // element counts (multiples of 4)
  int t;                     // segment number, >= 1
  float alpha;
};
hipError_t launch_segment_correct(const SegmentArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// attention coverage of a selection (mass and its per-head top-M bound)
// ---------------------------------------------------------------------------
struct MassArgs {
  Shape sh;
  int n_rows;               // query rows
  const int32_t* row_seq;   // nullable [n_rows]: cache sequence of each row (NULL: row r)
  const int32_t* row_len;   // [n_rows]: the row attends to positions 0..len-1
  const void* q;            // [n_rows, H_q, d]
  const void* k_cache;      // [*, cap, H_kv, d]
  const int32_t* idx;       // [n_rows, M] selected positions, -1 padded
  float scale;              // 1/sqrt(d)
  float* logits;            // workspace [n_rows * H_q, ld]
  int64_t ld;
  int32_t* lens;            // workspace [n_rows * H_q]: row lengths for the bound's select
  const int32_t* bidx;      // workspace [n_rows * H_q, M]: each head's own top-M
  float2* part;             // workspace [n_rows * H_q, part_ld]: (max, sum of exp) per 256-key block
  int64_t part_ld;
  float* mass;              // [n_rows, H_q]
  float* bound;             // nullable [n_rows, H_q]
};
// ---------------------------------------------------------------------------
// indexer training objective (per-row, per-head KL against the teacher)
// ---------------------------------------------------------------------------
struct KlArgs {
  Shape sh;
  int n;                    // prefill rows per sequence
  const void* q;            // [B, n, H_q, d] teacher queries
  const void* k_cache;      // [B, cap, H_kv, d] teacher keys (rows 0..n-1)
  const void* q_idx;        // [B, n, H_I, d_I]
  const void* k_idx;        // [B, cap, H_Ik, d_I]
  float scale;              // 1/sqrt(d)
  float* kl;                // [B, n, H_I]
  float* loss;              // nullable [1]: mean of kl
};
bool kl_mfma_supported(const Shape& sh);
hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t st);
hipError_t launch_indexer_kl_loss(const KlArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// indexer candidate dropout (top n_cand, random mask, the M best survivors)
// ---------------------------------------------------------------------------
struct DropoutArgs {
  int n_rows;
  int rows_per_seq;         // prefill: n (row r has length r % n + 1)
  int prefill;
  const int32_t* seq_lens;  // decode lengths
  const float* scores;      // [n_rows, ld]
  const float* u;           // [n_rows, ld] uniforms in [0, 1)
  int64_t ld;
  float p;                  // dropout ratio: candidate j survives iff u[j] >= p
  const uint32_t* mask;     // workspace [n_rows, mask_ld]: the top-n_cand bitmask
  int64_t mask_ld;
  int32_t* cnt;             // workspace [n_rows]: survivors per row
  float* cscore;            // workspace [n_rows, cld]: survivor scores in position order
  int32_t* cpos;            // workspace [n_rows, cld]: their positions
  int64_t cld;
  const int32_t* idx2;      // workspace [n_rows, M]: top-M entries of each survivor row
  int M;
  int32_t* idx_out;         // [n_rows, M]
};
hipError_t launch_dropout_compact(const DropoutArgs& a, hipStream_t st);
hipError_t launch_dropout_gather(const DropoutArgs& a, hipStream_t st);

int mass_key_blocks(int max_len);
hipError_t launch_mass_logits(const MassArgs& a, int max_len, hipStream_t st);
hipError_t launch_mass_reduce(const MassArgs& a, hipStream_t st);

hipError_t launch_attention(const AttnArgs& a, hipStream_t st);          // split kernel
hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t st);  // merge (nsplit > 1)
size_t attention_partial_floats(const Shape& sh, int n_rows, int nsplit);

// Decode with few sequences: selection and split attention in one launch
// (every split block selects the whole row; split partials as above).
bool select_attend_supported(const Shape& sh, int nsplit, int split_len);
// The shortest wide split (above 64 positions) with which a fused launch over
// `positions` selected entries fits, or 0.
int select_attend_wide_split(const Shape& sh, int positions);
hipError_t launch_select_attend(const AttnArgs& a, const SelectArgs& sa, hipStream_t st);
// the selection core of launch_select_attend alone (decode rows, full index lists)
hipError_t launch_select_runs(const SelectArgs& sa, hipStream_t st);


}  // namespace lisa
