/*
 * lisa.h - C ABI of the LISA (Linear-Indexed Sparse Attention) layer
 * library for AMD Instinct MI355X (gfx950).
 *
 * Method: "LISA: Linear-Indexed Sparse Attention for Efficient Long-Context
 * Reasoning" (arXiv 2607.19358v1), cited below as [LISA].  One attention
 * layer computes, for every query token t of every sequence b:
 *
 *   1. Indexer scores over the keys j = 0..t ([LISA] Section 3.2 Stage 2,
 *      the ReLU dot-product score defined under Eq. 2, summed over heads):
 *        s[t,j] = sum_{h < H_I} w_idx[h] * max(0, q_idx[t,h] . k_idx[j, h*H_Ik/H_I])
 *   2. Top-M selection: the min(M, t+1) keys with the largest s[t,j]; equal
 *      scores go to the later position, -0.0 equals +0.0 ([LISA] Section 3.2
 *      Stage 2, the top-M step that follows the summed indexer score).
 *   3. Sparse GQA softmax attention over the selected cached K/V rows, scale
 *      1/sqrt(d), query head h reading KV head h*H_kv/H_q ([LISA] Section
 *      3.1 Softmax Attention; Section 3.2 SA_M).
 *   4. Linear-attention branch with phi(x) = elu(x)+1 ([LISA] Section 3.1
 *      Linear Attention; Section 3.3 Eqs. 3-4, inclusive of token t):
 *        S_t = S_{t-1} + phi(k_lin[t])^T v_lin[t],  z_t = z_{t-1} + phi(k_lin[t])
 *        O_L[t] = phi(q_lin[t]) S_t / (phi(q_lin[t]) . z_t)
 *      (LISA_LINEAR_UNNORMALIZED: O_L[t] = phi(q_lin[t]) S_t, Eq. 4 as printed.)
 *   5. Gate ([LISA] Section 3.2 Eq. 1 and Section 3.3 Eq. 5), one scalar per
 *      token and query head:
 *        g[t,h] = sigmoid(x[t] . w_gate[:,h]),  out[t,h] = g*O_s[t,h] + (1-g)*O_L[t,h]
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major, contiguous, in device memory, and at
 *     least 16-byte aligned.  "T" means the activation dtype given by
 *     lisa_shape.dtype (fp32 or bf16); scores, S, z and w_idx are fp32.
 *   - Caches are token-major: k_cache/v_cache [B, cap, H_kv, d],
 *     k_idx_cache [B, cap, H_Ik, d_I].
 *   - Linear state S is [B, H_L, d, d] (row = phi(k) component, column = v
 *     component), z is [B, H_L, d].  w_gate is [hidden, H_q] (type T);
 *     w_idx is [H_I] (fp32).
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates or frees device memory and keeps no pointer after the
 *     work it enqueued has finished.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream): no host synchronisation, no device-to-host copies.  Results
 *     are deterministic (no floating-point atomics).  Calls that share a
 *     workspace must not overlap; calls with disjoint buffers may run on
 *     different streams at the same time.
 *   - Every call validates its arguments on the host before enqueuing
 *     anything.  On error it returns a negative status, enqueues nothing,
 *     modifies nothing, and lisa_last_error() describes the failure.
 *   - Device-side values (seq_lens) are not checked on the host: the caller
 *     guarantees 1 <= seq_lens[b] <= min(max_len, cap).
 */
#ifndef LISA_H
#define LISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LISA_OK                0
#define LISA_ERR_INVALID_ARG  -1   /* null pointer, inconsistent or out-of-range shape */
#define LISA_ERR_UNSUPPORTED  -2   /* valid but outside what the kernels implement */
#define LISA_ERR_WORKSPACE    -3   /* ws_bytes smaller than lisa_workspace_bytes() */
#define LISA_ERR_HIP          -4   /* a HIP launch or runtime call failed */

/* lisa_shape.dtype */
#define LISA_F32   0
#define LISA_BF16  1

/* lisa_shape.flags */
#define LISA_LINEAR_UNNORMALIZED  1u   /* O_L = phi(q) S, no normaliser z */
/* Sliding-window attention ([LISA] Section 3.2 Stage 1, Eq. 1: a fixed budget
 * of the M most recent tokens): query t attends to positions
 * max(0, t+1-M)..t, the indexer does not run, and the indexer arguments
 * (q_idx, k_idx_new, k_idx_cache, w_idx) are neither read nor written and may
 * be NULL.  idx_out, if given, receives those positions.  Decode and prefill
 * only. */
#define LISA_SLIDING_WINDOW       2u

/* op codes for lisa_workspace_bytes() */
#define LISA_OP_DECODE           0
#define LISA_OP_PREFILL          1
#define LISA_OP_TOPK_DECODE      2
#define LISA_OP_TOPK_PREFILL     3
#define LISA_OP_LINEAR_UPDATE    4
#define LISA_OP_DENSE_DECODE     5
#define LISA_OP_MASS             6
#define LISA_OP_DROPOUT_DECODE   7
#define LISA_OP_DROPOUT_PREFILL  8

/* rows_mode of lisa_indexer_topk() */
#define LISA_ROWS_DECODE   0
#define LISA_ROWS_PREFILL  1

typedef struct lisa_shape {
  int32_t B;        /* batch (sequences)                                         */
  int32_t H_q;      /* query heads                                               */
  int32_t H_kv;     /* key/value heads; H_q % H_kv == 0                          */
  int32_t d;        /* head dimension of q, k, v and of the linear branch        */
  int32_t H_I;      /* indexer query heads                                       */
  int32_t H_Ik;     /* indexer key heads; H_I % H_Ik == 0 (H_Ik = 1: shared key) */
  int32_t d_I;      /* indexer head dimension                                    */
  int32_t H_L;      /* linear-attention heads; must equal H_q                    */
  int32_t hidden;   /* width of the gate input x                                 */
  int32_t M;        /* top-M budget, >= 1                                        */
  int32_t cap;      /* cache capacity: rows per sequence in every cache          */
  int32_t max_len;  /* decode: upper bound of seq_lens[b]; prefill: unused (0)   */
  int32_t chunk;    /* prefill chunk of the linear scan (64; 0 selects 64)       */
  int32_t dtype;    /* LISA_F32 or LISA_BF16                                     */
  uint32_t flags;   /* LISA_LINEAR_UNNORMALIZED | LISA_SLIDING_WINDOW, or 0      */
} lisa_shape;
/* Counts beyond B = 65536, cap or M = 2^26, hidden = 2^20, H_q or H_I = 1024
 * or d_I = 4096 are rejected with LISA_ERR_UNSUPPORTED. */

/*
 * Bytes of workspace an operation needs.  `n` is the prefill length (tokens
 * per sequence) for LISA_OP_PREFILL / LISA_OP_TOPK_PREFILL, the token count
 * for LISA_OP_LINEAR_UPDATE and the number of query rows for LISA_OP_MASS,
 * and the prefill length for LISA_OP_DROPOUT_PREFILL; it is ignored
 * otherwise.  Returns 0 for an
 * invalid shape or op (lisa_last_error() says why).
 */
size_t lisa_workspace_bytes(const lisa_shape* shape, int op, int32_t n);

/*
 * One decode step ([LISA] Section 3.2 Stage 2: at each generation step the
 * indexer scores the context, M tokens feed the sparse attention, which with
 * the linear state produces the step's output; the new token then enters the
 * linear state and the KV cache).
 *
 * seq_lens  [B] int32, device: L_b, the context length INCLUDING the new token.
 * q         [B, H_q, d] T        k_new, v_new [B, H_kv, d] T
 * q_idx     [B, H_I, d_I] T      k_idx_new    [B, H_Ik, d_I] T
 * q_lin, k_lin, v_lin [B, H_L, d] T
 * x         [B, hidden] T        w_gate [hidden, H_q] T     w_idx [H_I] fp32
 * k_cache, v_cache, k_idx_cache: rows 0..L_b-2 hold the history; the call
 *           writes the new token into row L_b-1 (in place).
 * S, z      in: state after L_b-1 tokens; out: state after L_b tokens (in place).
 * out       [B, H_q, d] T.
 * idx_out   nullable [B, M] int32: ascending selected positions, -1 padded.
 * ws        workspace of lisa_workspace_bytes(shape, LISA_OP_DECODE, 0) bytes.
 * With M >= max_len every position is selected whatever the scores, so the
 * step appends k_idx_new but reads neither q_idx, w_idx nor the cached index
 * keys (they must still be valid pointers); the results are those of the
 * full selection.
 */
int lisa_decode_step(const lisa_shape* shape, const int32_t* seq_lens,
                     const void* q, const void* k_new, const void* v_new,
                     const void* q_idx, const void* k_idx_new,
                     const void* q_lin, const void* k_lin, const void* v_lin,
                     const void* x, const void* w_gate, const float* w_idx,
                     void* k_cache, void* v_cache, void* k_idx_cache,
                     float* S, float* z, void* out, int32_t* idx_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * The same decode step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): its workspace is a static device array of
 * LISA_DECODE_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing and frees nothing.  Arguments and
 * results are those of lisa_decode_step without ws/ws_bytes; a shape whose
 * lisa_workspace_bytes(shape, LISA_OP_DECODE, 0) exceeds
 * LISA_DECODE_SCRATCH_BYTES is rejected with LISA_ERR_WORKSPACE (4 MiB
 * covers batch 1 at contexts up to 16K with M = 2048 for a 28/4-head,
 * d = 128 layer).  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (nothing in it has to start at zero): calls that
 * overlap on one GPU, e.g. on two streams, race and must not be made.
 */
#define LISA_DECODE_SCRATCH_BYTES ((size_t)4 << 20)
int lisa_decode_step_noalloc(const lisa_shape* shape, const int32_t* seq_lens,
                             const void* q, const void* k_new, const void* v_new,
                             const void* q_idx, const void* k_idx_new,
                             const void* q_lin, const void* k_lin, const void* v_lin,
                             const void* x, const void* w_gate, const float* w_idx,
                             void* k_cache, void* v_cache, void* k_idx_cache,
                             float* S, float* z, void* out, int32_t* idx_out, void* stream);

/*
 * Causal prefill of n tokens in every sequence (positions 0..n-1): steps 1-5
 * above for every row t < n ([LISA] Section 3.2 Stages 1-2 for the indexer,
 * the selection and SA_M; Section 3.3 Eqs. 3-5 for the linear branch as a
 * chunked causal scan and the gate).  Rows with t + 1 <= M take every key.
 *
 * q         [B, n, H_q, d] T
 * k_cache, v_cache [B, cap, H_kv, d] T, k_idx_cache [B, cap, H_Ik, d_I] T:
 *           rows 0..n-1 hold this prefill's keys/values (written by the
 *           caller; read only here).  n <= cap.
 * q_idx     [B, n, H_I, d_I] T
 * q_lin, k_lin, v_lin [B, n, H_L, d] T     x [B, n, hidden] T
 * w_gate    [hidden, H_q] T      w_idx [H_I] fp32
 * S, z      in: S_0, z_0; out: the state after the n tokens (in place).
 * out       [B, n, H_q, d] T
 * idx_out   nullable [B, n, M] int32: per row, ascending positions, -1 padded.
 * ws        workspace of lisa_workspace_bytes(shape, LISA_OP_PREFILL, n) bytes.
 * The gate and the linear branch run on an internal side stream next to the
 * indexer and the select, forked from and joined back into `stream` with
 * events, so the call keeps the ordering of `stream` and can be captured in
 * a graph.  The library creates one side stream and two events per device
 * and caller stream on the first call outside a capture, and keeps them
 * until the process ends; it creates at most 32 such pairs in a process.
 * Without one (the first call made inside a capture, more than 32 caller
 * streams, sliding-window mode), everything runs on `stream`.
 */
int lisa_prefill(const lisa_shape* shape, int32_t n,
                 const void* q, const void* k_cache, const void* v_cache,
                 const void* k_idx_cache, const void* q_idx,
                 const void* q_lin, const void* k_lin, const void* v_lin,
                 const void* x, const void* w_gate, const float* w_idx,
                 float* S, float* z, void* out, int32_t* idx_out,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Indexer scores and top-M selection alone ([LISA] Section 3.2 Stage 2).
 *
 * rows_mode LISA_ROWS_DECODE: one row per sequence b, of length
 *   seq_lens[b] (device, [B]); q_idx [B, H_I, d_I]; keys are rows
 *   0..seq_lens[b]-1 of k_idx_cache (no append).  scores are [B, scores_ld].
 *   idx_out [B, M].
 * rows_mode LISA_ROWS_PREFILL: n rows per sequence, row t of length t+1;
 *   seq_lens is ignored (may be NULL); q_idx [B, n, H_I, d_I]; scores are
 *   [B, n, scores_ld]; idx_out [B, n, M].
 * scores_in  nullable: when set, the call skips scoring and selects from these
 *            fp32 rows (q_idx, k_idx_cache and w_idx may then be NULL).
 * scores_out nullable: when set (and scores_in is NULL), receives the fp32
 *            scores of each row's positions 0..len-1; other entries untouched.
 * scores_ld  row stride in elements of scores_in/out: a multiple of 4 and
 *            >= the longest row.
 * idx_out    ascending selected positions, -1 padded.
 * ws         workspace of lisa_workspace_bytes(shape, LISA_OP_TOPK_DECODE or
 *            LISA_OP_TOPK_PREFILL, n) bytes.
 */
int lisa_indexer_topk(const lisa_shape* shape, int rows_mode, int32_t n,
                      const int32_t* seq_lens, const void* q_idx,
                      const void* k_idx_cache, const float* w_idx,
                      const float* scores_in, int64_t scores_ld,
                      float* scores_out, int32_t* idx_out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Segment state correction at the end of segment t ([LISA] Section 3.3
 * "Segment State Update", Eqs. 6-9), elementwise over S [B, H_L, d, d] and
 * z [B, H_L, d] (fp32, device, 16-byte aligned):
 *   grad      = S - S_start                        (Eq. 6)
 *   corrected = (1 - alpha) grad + alpha mean      (Eq. 8; mean = 0 when t == 1)
 *   S         = S_start + corrected                (Eq. 9)
 *   mean      = mean + (grad - mean) / t           (Eq. 7: the mean of the raw
 *                                                   directions of segments 1..t)
 *   S_start   = S                                  (where segment t+1 starts)
 * and the same for z with z_start and mean_z (the normaliser is part of the
 * state).  S, z: in, the state reached at the segment's end; out, corrected.
 * S_start, z_start: in, the state at the segment's start; out, the corrected
 * state.  mean_S, mean_z: in, the mean direction of segments 1..t-1 (not
 * read when t == 1); out, of segments 1..t.  t >= 1 counts segments of k
 * tokens; the caller calls this after every k tokens (decode steps or
 * prefill chunks); alpha must be finite.  d must be a multiple of 4.  Nothing is allocated; the
 * call is asynchronous on `stream`.
 */
int lisa_segment_correct(const lisa_shape* shape, float* S, float* z, float* S_start, float* z_start,
                         float* mean_S, float* mean_z, int32_t t, float alpha, void* stream);

/*
 * Linear-state update over n_tokens tokens ([LISA] Section 3.3 Eq. 3):
 *   S += sum_t phi(k_lin[t])^T v_lin[t],  z += sum_t phi(k_lin[t]).
 * k_lin, v_lin [B, n_tokens, H_L, d] T; S [B, H_L, d, d], z [B, H_L, d] fp32.
 */
int lisa_linear_state_update(const lisa_shape* shape, int32_t n_tokens,
                             const void* k_lin, const void* v_lin,
                             float* S, float* z, void* stream);

/*
 * Dense baseline: full causal GQA softmax attention of one new token per
 * sequence over cache rows 0..seq_lens[b]-1 (no indexer, no linear branch,
 * no gate, no append: row seq_lens[b]-1 must already hold the new k, v).
 * q [B, H_q, d] T; out [B, H_q, d] T.  This is the M >= n case of step 3.
 */
int lisa_dense_decode(const lisa_shape* shape, const int32_t* seq_lens,
                      const void* q, const void* k_cache, const void* v_cache,
                      void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Attention coverage of a selection ([LISA] Section 4, "Optimal Window Size
 * M and Attention Coverage", Eq. 10).  For query row r and query head h
 * (KV head g = h H_kv / H_q), with dense weights
 *   a_j = exp(q[r, h] . k[j, g] / sqrt(d)),  j = 0 .. row_len[r]-1,
 *   mass[r, h]  = sum over the positions in idx[r, :] of a_j / sum_j a_j
 *   bound[r, h] = sum of the M largest a_j / sum_j a_j
 * The bound is the coverage of the head's own best M positions, which no
 * set of M positions shared by the heads can exceed.
 *
 * n_rows   query rows, 0 <= n_rows <= 65535 (0: nothing is enqueued).
 * row_seq  nullable [n_rows] int32, device: the cache sequence of row r
 *          (NULL: sequence r).  Several rows may share a sequence, e.g.
 *          sampled prefill rows.
 * row_len  [n_rows] int32, device: the row attends to cache rows
 *          0 .. row_len[r]-1 (its own key included); 1 <= row_len[r] <=
 *          shape.max_len <= cap (not checked on the device).
 * q        [n_rows, H_q, d] T.       k_cache [*, cap, H_kv, d] T.
 * idx      [n_rows, M] int32: distinct positions (any order); entries
 *          outside [0, row_len[r]), such as the -1 padding, are skipped.
 *          The idx_out of lisa_decode_step or lisa_prefill fits as it is.
 * mass     [n_rows, H_q] fp32.       bound  nullable [n_rows, H_q] fp32.
 * ws       workspace of lisa_workspace_bytes(shape, LISA_OP_MASS, n_rows)
 *          bytes (fp32 logits of every row and head, the bound's index sets).
 * shape.B is not used; shape.M is the budget of the bound; every other
 * field as for lisa_decode_step.  Asynchronous on `stream`.
 */
int lisa_attention_mass(const lisa_shape* shape, int32_t n_rows, const int32_t* row_seq,
                        const int32_t* row_len, const void* q, const void* k_cache,
                        const int32_t* idx, float* mass, float* bound,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Indexer training objective ([LISA] Section 3.2 Stage 2, Eq. 2), forward
 * only, over the n prefill rows of every sequence.  For row t and indexer
 * head j, over the keys k = 0..t:
 *   S_k  = max(0, q_idx[t, j] . k_idx[k, j H_Ik / H_I])     (no head weight)
 *   Q    = softmax(S)
 *   T    = mean over the teacher heads h = j G_T .. (j+1) G_T - 1,
 *          G_T = H_q / H_I, of softmax_k(q[t, h] . k[k, h H_kv / H_q] / sqrt(d))
 *          (the sum of the teacher rows renormalised)
 *   kl_out[b, t, j] = KL(T || Q) = sum_k T_k (ln T_k - ln Q_k)
 *   loss_out[0]     = the mean of kl_out over b, t and j          (Eq. 2)
 * The teacher is the layer's own full attention: q [B, n, H_q, d] and
 * k_cache [B, cap, H_kv, d] (rows 0..n-1); q_idx [B, n, H_I, d_I] and
 * k_idx_cache [B, cap, H_Ik, d_I] (rows 0..n-1) are the indexer's.
 * kl_out [B, n, H_I] fp32; loss_out nullable [1] fp32.  Requires H_q to be a
 * multiple of H_I.  bf16 with d = 128, d_I = 64 and each teacher group inside
 * one KV head runs on the matrix cores; other shapes run a slower vector
 * kernel.  No workspace; asynchronous on `stream`.
 */
int lisa_indexer_kl(const lisa_shape* shape, int32_t n, const void* q, const void* k_cache,
                    const void* q_idx, const void* k_idx_cache, float* kl_out, float* loss_out,
                    void* stream);

/*
 * Indexer candidate dropout ([LISA] Section 3.2 Stage 2: early in training
 * the top 1.2 M candidates are taken and a random 20% of them masked out
 * before the sparse attention is filled; the ratio is lowered over
 * training).  Per score row of length len:
 *   1. candidates: the top min(len, n_cand) positions (order as for top-M:
 *      score descending, ties to the later position, -0.0 == +0.0);
 *   2. candidate j survives iff u[j] >= p (u: the caller's uniform draws in
 *      [0, 1), one per position, same layout as the scores);
 *   3. idx_out: the min(M, #survivors) best survivors in that order,
 *      ascending, -1 padded.
 * rows_mode, n, seq_lens and the score layout as for lisa_indexer_topk
 * (prefill rows: row t of each sequence has length t+1, scores
 * [B, n, scores_ld]; decode: [B, scores_ld]); scores_ld a multiple of 4 and
 * at least the longest row.  Scores must be finite and above -FLT_MAX.
 * n_cand >= 1 (the paper's 1.2 M is ceil(1.2 M)); p is the dropout ratio
 * (p <= 0 keeps every candidate, p > 1 none).  idx_out [rows, M] int32.
 * ws: lisa_workspace_bytes(shape, LISA_OP_DROPOUT_DECODE, 0) or
 * lisa_workspace_bytes(shape, LISA_OP_DROPOUT_PREFILL, n) bytes, which
 * covers any n_cand (the top-n_cand bitmask, each row's survivors as a short
 * row of scores and positions, and their top-M); a smaller n_cand needs
 * less, and a workspace short of what the given n_cand needs is rejected.
 * Asynchronous on `stream`.
 */
int lisa_candidate_dropout(const lisa_shape* shape, int rows_mode, int32_t n, const int32_t* seq_lens,
                           const float* scores, const float* u, int64_t scores_ld, int32_t n_cand,
                           float p, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* Text of a status code. */
const char* lisa_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* lisa_last_error(void);

/*
 * Kernel timing hook (measurement only).  lisa_timing_enable(k, starts,
 * stops, n) makes the next n launches of kernel k, on the calling host
 * thread, go through hipExtLaunchKernel with the given hipEvent_t pairs, so
 * each pair brackets that kernel's own dispatch (the interval a kernel trace
 * reports, without launch gaps).  Before each such launch the library waits
 * on the host for the stream's earlier work, so that the pair does not also
 * cover the tail of the kernel before it.  lisa_timing_count() returns how
 * many pairs were used so far; lisa_timing_enable(k, NULL, NULL, 0) disables
 * it.  Not for use under stream capture.  Kernel ids are listed by
 * lisa_kernel_name().
 */
int lisa_timing_enable(int kernel_id, void** start_events, void** stop_events, int n);
int lisa_timing_count(void);
const char* lisa_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* LISA_H */
