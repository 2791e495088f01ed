// C-ABI host layer of the LISA library: argument validation, workspace
// layout, launch sequencing, error state and the kernel timing hook.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "lisa.h"
#include "lisa_kernels.h"
#include "lisa_prefill.h"

using namespace lisa;

// Workspace of lisa_decode_step_noalloc (see decode_scratch below).
static __device__ __align__(256) unsigned char scratch[LISA_DECODE_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(LISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int MAX_ROW = 65536;  // longest score row the select kernel holds

// ---------------------------------------------------------------------------
// shape validation
// ---------------------------------------------------------------------------
int check_shape(const lisa_shape* s, Shape& o) {
  if (!s) return fail(LISA_ERR_INVALID_ARG, "shape is NULL");
  if (s->dtype != LISA_F32 && s->dtype != LISA_BF16) return fail(LISA_ERR_INVALID_ARG, "dtype %d", s->dtype);
  if (s->flags & ~(LISA_LINEAR_UNNORMALIZED | LISA_SLIDING_WINDOW))
    return fail(LISA_ERR_INVALID_ARG, "unknown flags 0x%x", s->flags);
  if (s->B < 1 || s->H_q < 1 || s->H_kv < 1 || s->d < 1 || s->H_I < 1 || s->H_Ik < 1 || s->d_I < 1 ||
      s->H_L < 1 || s->hidden < 1 || s->M < 1 || s->cap < 1)
    return fail(LISA_ERR_INVALID_ARG, "every count must be >= 1");
  // upper bounds that keep every size and index computation of the library
  // inside its integer types
  if (s->B > (1 << 16) || s->cap > (1 << 26) || s->M > (1 << 26) || s->hidden > (1 << 20) || s->H_q > (1 << 10) ||
      s->H_I > (1 << 10) || s->d_I > (1 << 12))
    return fail(LISA_ERR_UNSUPPORTED, "a count is too large (B <= 65536, cap and M <= 2^26, hidden <= 2^20, "
                                      "H_q and H_I <= 1024, d_I <= 4096)");
  if (s->H_q % s->H_kv) return fail(LISA_ERR_INVALID_ARG, "H_q %% H_kv != 0");
  if (s->H_I % s->H_Ik) return fail(LISA_ERR_INVALID_ARG, "H_I %% H_Ik != 0");
  if (s->H_L != s->H_q) return fail(LISA_ERR_INVALID_ARG, "H_L (%d) must equal H_q (%d)", s->H_L, s->H_q);
  if (s->chunk != 0 && s->chunk != 64) return fail(LISA_ERR_UNSUPPORTED, "chunk %d (64 only)", s->chunk);
  if (s->d != 32 && s->d != 64 && s->d != 128) return fail(LISA_ERR_UNSUPPORTED, "head dim %d", s->d);
  if (s->H_q / s->H_kv > 8) return fail(LISA_ERR_UNSUPPORTED, "more than 8 query heads per KV head");
  if (s->H_q > 64) return fail(LISA_ERR_UNSUPPORTED, "more than 64 query heads");
  const int R = s->H_I / s->H_Ik;
  if (R != 1 && R != 2 && R != 4) return fail(LISA_ERR_UNSUPPORTED, "H_I / H_Ik = %d", R);
  const int VEC = s->dtype == LISA_F32 ? 4 : 8;
  if (s->d_I % VEC || !is_pow2(s->d_I / VEC) || !is_pow2(s->H_Ik) || s->H_Ik * s->d_I / VEC > 64)
    return fail(LISA_ERR_UNSUPPORTED, "index key row H_Ik*d_I = %d", s->H_Ik * s->d_I);
  o.B = s->B; o.H_q = s->H_q; o.H_kv = s->H_kv; o.d = s->d; o.H_I = s->H_I; o.H_Ik = s->H_Ik;
  o.d_I = s->d_I; o.H_L = s->H_L; o.hidden = s->hidden; o.M = s->M; o.cap = s->cap;
  o.max_len = s->max_len; o.chunk = s->chunk ? s->chunk : 64; o.dtype = s->dtype; o.flags = s->flags;
  return LISA_OK;
}

int check_decode_len(const Shape& sh) {
  if (sh.max_len < 1 || sh.max_len > sh.cap)
    return fail(LISA_ERR_INVALID_ARG, "max_len %d outside [1, cap=%d]", sh.max_len, sh.cap);
  if (sh.max_len > MAX_ROW) return fail(LISA_ERR_UNSUPPORTED, "max_len %d > %d", sh.max_len, MAX_ROW);
  return LISA_OK;
}

int check_prefill_len(const Shape& sh, int n) {
  if (n < 1 || n > sh.cap) return fail(LISA_ERR_INVALID_ARG, "n %d outside [1, cap=%d]", n, sh.cap);
  if (n > MAX_ROW) return fail(LISA_ERR_UNSUPPORTED, "n %d > %d", n, MAX_ROW);
  return LISA_OK;
}

#define REQUIRE_PTR(p)                                                                   \
  do {                                                                                   \
    if (!(p)) return fail(LISA_ERR_INVALID_ARG, "%s is NULL", #p);                      \
    if (!aligned16(p)) return fail(LISA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)
#define OPTIONAL_PTR(p)                                                                      \
  do {                                                                                       \
    if ((p) && !aligned16(p)) return fail(LISA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

// ---------------------------------------------------------------------------
// workspace layouts
// ---------------------------------------------------------------------------
int64_t decode_scores_ld(const Shape& sh) { return (int64_t)align_up((size_t)sh.max_len, 64); }

void decode_split(const Shape& sh, int positions, int& nsplit, int& split_len) {
  int sl = 64;
  while ((positions + sl - 1) / sl > 32) sl *= 2;
  // with many blocks, 128 positions per split keep all four waves of a
  // gather block busy (32 entries each per round)
  if ((size_t)sh.B * sh.H_kv * ((positions + sl - 1) / sl) > 1024 && sl < 128) sl = 128;
  while ((size_t)sh.B * sh.H_kv * ((positions + sl - 1) / sl) > 4096 && sl < positions) sl *= 2;
  split_len = sl;
  nsplit = (positions + sl - 1) / sl;
}

int decode_gate_chunks(const Shape& sh) { return (sh.hidden + 63) / 64; }

struct DecodeWs {
  size_t scores, idx, o_lin, lin_den, gate, part, total;
  int nsplit, split_len;
};

// A decode step of few sequences selects inside its attention launch (every
// attention block selects the whole row, then attends to its split); larger
// batches run a separate select launch.  lisa_indexer_topk routes decode rows
// the same way, so it selects with the core the decode step of that shape
// uses.
bool decode_fused(const Shape& sh, int nsplit, int split_len) {
  return select_attend_supported(sh, nsplit, split_len);
}

// Splits of the decode step's attention: decode_split's, or, where those
// would take more fused select + attention blocks than the chip runs at once
// (one per CU), the shortest wide split that fits the fused launch.
void decode_step_split(const Shape& sh, int& nsplit, int& split_len) {
  const int positions = sh.M < sh.max_len ? sh.M : sh.max_len;
  decode_split(sh, positions, nsplit, split_len);
  if ((sh.flags & LISA_SLIDING_WINDOW) || sh.M >= sh.max_len || decode_fused(sh, nsplit, split_len)) return;
  const int wide = select_attend_wide_split(sh, positions);
  if (wide) {
    split_len = wide;
    nsplit = (positions + wide - 1) / wide;
  }
}

DecodeWs decode_ws(const Shape& sh) {
  DecodeWs w;
  Layout L;
  decode_step_split(sh, w.nsplit, w.split_len);
  w.scores = L.take((size_t)sh.B * decode_scores_ld(sh) * 4);
  w.idx = L.take((size_t)sh.B * sh.M * 4);
  w.o_lin = L.take((size_t)sh.B * sh.H_L * sh.d * 4);
  w.lin_den = L.take((size_t)sh.B * sh.H_L * 4);
  w.gate = L.take((size_t)sh.B * decode_gate_chunks(sh) * sh.H_q * 4);
  w.part = L.take(attention_partial_floats(sh, sh.B, w.nsplit) * 4);
  w.total = L.off;
  return w;
}

struct DenseWs {
  size_t part, total;
  int nsplit, split_len;
};

DenseWs dense_ws(const Shape& sh) {
  DenseWs w;
  Layout L;
  decode_split(sh, sh.max_len, w.nsplit, w.split_len);
  w.part = L.take(attention_partial_floats(sh, sh.B, w.nsplit) * 4);
  w.total = L.off;
  return w;
}

int64_t prefill_scores_ld(int n) { return (int64_t)align_up((size_t)n, 64); }

struct PrefillWs {
  size_t scores, idx, mask, occ, o_lin, gate, w_t, z_tmp, seg, total;
};

// Key-tile occupancy of the prefill bitmask: one row of words per 32 query
// rows, one bit per key tile of 64.
int64_t prefill_occ_ld(int n) { return (int64_t)(((n + 63) / 64 + 31) / 32); }
size_t prefill_occ_words(const Shape& sh, int n) { return (size_t)sh.B * ((n + 31) / 32) * prefill_occ_ld(n); }

PrefillWs prefill_ws(const Shape& sh, int n) {
  PrefillWs w;
  Layout L;
  const int srows = n > sh.M ? n - sh.M : 0;
  const bool mfma_attn = attn_mfma_supported(sh);
  w.scores = L.take((size_t)sh.B * srows * prefill_scores_ld(n) * 4);
  w.idx = L.take(mfma_attn ? 0 : (size_t)sh.B * n * sh.M * 4);  // the MFMA path reads the bitmask
  w.mask = L.take(mfma_attn ? (size_t)sh.B * n * attn_mask_ld(n) * 4 : 0);
  w.occ = L.take(mfma_attn ? prefill_occ_words(sh, n) * 4 : 0);
  w.o_lin = L.take((size_t)sh.B * n * sh.H_L * sh.d * 4);
  w.gate = L.take((size_t)sh.B * n * sh.H_q * 4);
  w.w_t = L.take(gate_mfma_supported(sh) ? gate_transpose_elems(sh) * 2 : 0);
  w.z_tmp = L.take((size_t)sh.B * sh.H_L * sh.d * 4);
  w.seg = L.take(linear_mfma_supported(sh) ? linear_seg_floats(sh, n) * 4 : 0);
  w.total = L.off;
  return w;
}

struct MassWs {
  size_t logits, lens, bidx, part, total;
};

int64_t mass_logits_ld(const Shape& sh) { return (int64_t)align_up((size_t)sh.max_len, 64); }

MassWs mass_ws(const Shape& sh, int n_rows) {
  MassWs w;
  Layout L;
  const size_t rows = (size_t)n_rows * sh.H_q;
  w.logits = L.take(rows * mass_logits_ld(sh) * 4);
  w.lens = L.take(rows * 4);
  w.bidx = L.take(rows * sh.M * 4);
  w.part = L.take(rows * mass_key_blocks(sh.max_len) * 8);
  w.total = L.off;
  return w;
}

struct DropoutWs {
  size_t mask, cnt, cscore, cpos, idx2, total;
};

// Survivor rows hold at most min(n_cand, longest) entries; the workspace
// query sizes them for the longest row (any n_cand).
int64_t dropout_cld(int cmax) { return (int64_t)align_up((size_t)cmax, 64); }
int64_t dropout_mask_ld(int longest) { return (longest + 31) / 32; }

DropoutWs dropout_ws(const Shape& sh, int64_t rows, int longest, int cmax) {
  DropoutWs w;
  Layout L;
  w.mask = L.take((size_t)rows * dropout_mask_ld(longest) * 4);
  w.cnt = L.take((size_t)rows * 4);
  w.cscore = L.take((size_t)rows * dropout_cld(cmax) * 4);
  w.cpos = L.take((size_t)rows * dropout_cld(cmax) * 4);
  w.idx2 = L.take((size_t)rows * sh.M * 4);
  w.total = L.off;
  return w;
}

struct TopkWs {
  size_t scores, total;
};

TopkWs topk_ws(const Shape& sh, int rows_mode, int n) {
  TopkWs w;
  Layout L;
  if (rows_mode == LISA_ROWS_DECODE) {
    w.scores = L.take((size_t)sh.B * decode_scores_ld(sh) * 4);
  } else {
    const int srows = n > sh.M ? n - sh.M : 0;
    w.scores = L.take((size_t)sh.B * srows * prefill_scores_ld(n) * 4);
  }
  w.total = L.off;
  return w;
}

template <typename P> P* at(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(ws) + off); }

// ---------------------------------------------------------------------------
// side streams: a prefill forks its linear branch and gate onto a second
// stream (default priority, non-blocking) that joins back before the
// attention, so they overlap the indexer and the select.  One side stream
// and event pair per (device, caller stream), created on first use outside
// a graph capture and kept until the process ends; at most
// kMaxSideStreams of them exist.  While none exists for a caller stream
// (table full, capture, or creation failed) the work stays on the caller's
// stream, which changes the timing only.
// ---------------------------------------------------------------------------
constexpr size_t kMaxSideStreams = 32;

struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

SideStream* side_stream(hipStream_t caller) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, SideStream> table;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = table.find({dev, caller});
  if (it != table.end()) return &it->second;
  if (table.size() >= kMaxSideStreams) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  SideStream ss;
  if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
  if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
    if (ss.fork) (void)hipEventDestroy(ss.fork);
    (void)hipStreamDestroy(ss.s);
    return nullptr;
  }
  return &(table[{dev, caller}] = ss);
}

// ---------------------------------------------------------------------------
// timing hook
// ---------------------------------------------------------------------------
struct Timing {
  int kid = -1;
  hipEvent_t* starts = nullptr;
  hipEvent_t* stops = nullptr;
  int n = 0;
  int count = 0;
} g_timing;

const char* const kKernelNames[KID_COUNT] = {
    "decode_phase_a", "topm_select", "gather_attention", "prefill_index_scores", "prefill_gate",
    "prefill_linear", "prefill_attention", "linear_state_update", "attention_combine",
    "prefill_linear_sums", "prefill_linear_prefix", "prefill_gate_transpose", "select_attention",
    "segment_correct", "mass_logits", "mass_select", "mass_reduce", "indexer_kl", "candidate_dropout_compact",
    "prefill_tile_occupancy"};

thread_local LaunchEvents g_next_launch;

bool timing_on(int kid) { return g_timing.kid == kid && g_timing.count < g_timing.n; }
bool timing_armed() { return g_timing.kid >= 0 && g_timing.count < g_timing.n; }

// A timed launch hands its event pair to the kernel's own dispatch
// (hipExtLaunchKernel); the pair counts once the launcher has consumed it.
#define LAUNCH(kid, st, call)                                                       \
  do {                                                                              \
    const bool timed_ = timing_on(kid);                                             \
    if (timed_) {                                                                   \
      (void)hipStreamSynchronize(st); /* the pair times this kernel alone */        \
      next_launch_events().start = g_timing.starts[g_timing.count];                 \
      next_launch_events().stop = g_timing.stops[g_timing.count];                   \
    }                                                                               \
    const hipError_t e_ = (call);                                                   \
    if (timed_) {                                                                   \
      if (!next_launch_events().start) ++g_timing.count;                            \
      next_launch_events() = LaunchEvents();                                        \
    }                                                                               \
    if (e_ != hipSuccess) return fail_hip(e_, kKernelNames[kid]);                   \
  } while (0)

// ---------------------------------------------------------------------------
// static scratch of the allocation-free decode step: one copy per GPU, held
// until the process ends.  Host code reaches it only through the device
// address that hipGetSymbolAddress returns on each device.
// ---------------------------------------------------------------------------
constexpr int MAX_DEVICES = 64;

int decode_scratch(void*& ptr) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "decode scratch: hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(LISA_ERR_UNSUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "decode scratch address");
    addr[dev] = p;
  }
  ptr = addr[dev];
  return LISA_OK;
}

int decode_step(const Shape& sh, const int32_t* seq_lens, const void* q, const void* k_new, const void* v_new,
                const void* q_idx, const void* k_idx_new, const void* q_lin, const void* k_lin, const void* v_lin,
                const void* x, const void* w_gate, const float* w_idx, void* k_cache, void* v_cache,
                void* k_idx_cache, float* S, float* z, void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                void* stream);
int decode_check_pointers(const Shape& sh, const int32_t* seq_lens, const void* q, const void* k_new,
                          const void* v_new, const void* q_idx, const void* k_idx_new, const void* q_lin,
                          const void* k_lin, const void* v_lin, const void* x, const void* w_gate,
                          const float* w_idx, void* k_cache, void* v_cache, void* k_idx_cache, float* S, float* z,
                          void* out, int32_t* idx_out);

}  // namespace

LaunchEvents& lisa::next_launch_events() { return g_next_launch; }

// ===========================================================================
// exported entry points
// ===========================================================================
extern "C" {

const char* lisa_status_string(int status) {
  switch (status) {
    case LISA_OK: return "ok";
    case LISA_ERR_INVALID_ARG: return "invalid argument";
    case LISA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LISA_ERR_WORKSPACE: return "workspace too small";
    case LISA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* lisa_last_error(void) { return g_err.c_str(); }

const char* lisa_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= KID_COUNT) return nullptr;
  return kKernelNames[kernel_id];
}

int lisa_timing_enable(int kernel_id, void** start_events, void** stop_events, int n) {
  if (n == 0) {
    g_timing = Timing();
    return LISA_OK;
  }
  if (kernel_id < 0 || kernel_id >= KID_COUNT || !start_events || !stop_events || n < 0)
    return fail(LISA_ERR_INVALID_ARG, "bad timing request");
  g_timing.kid = kernel_id;
  g_timing.starts = reinterpret_cast<hipEvent_t*>(start_events);
  g_timing.stops = reinterpret_cast<hipEvent_t*>(stop_events);
  g_timing.n = n;
  g_timing.count = 0;
  return LISA_OK;
}

int lisa_timing_count(void) { return g_timing.count; }

size_t lisa_workspace_bytes(const lisa_shape* shape, int op, int32_t n) {
  Shape sh;
  if (check_shape(shape, sh) != LISA_OK) return 0;
  switch (op) {
    case LISA_OP_DECODE:
      if (check_decode_len(sh) != LISA_OK) return 0;
      return decode_ws(sh).total;
    case LISA_OP_DENSE_DECODE:
      if (check_decode_len(sh) != LISA_OK) return 0;
      return dense_ws(sh).total;
    case LISA_OP_PREFILL:
      if (check_prefill_len(sh, n) != LISA_OK) return 0;
      return prefill_ws(sh, n).total;
    case LISA_OP_TOPK_DECODE:
      if (check_decode_len(sh) != LISA_OK) return 0;
      return topk_ws(sh, LISA_ROWS_DECODE, 0).total;
    case LISA_OP_TOPK_PREFILL:
      if (check_prefill_len(sh, n) != LISA_OK) return 0;
      return topk_ws(sh, LISA_ROWS_PREFILL, n).total;
    case LISA_OP_MASS:
      if (check_decode_len(sh) != LISA_OK || n < 1) return 0;
      return mass_ws(sh, n).total;
    case LISA_OP_DROPOUT_DECODE:
      if (check_decode_len(sh) != LISA_OK) return 0;
      return dropout_ws(sh, sh.B, sh.max_len, sh.max_len).total;
    case LISA_OP_DROPOUT_PREFILL:
      if (check_prefill_len(sh, n) != LISA_OK) return 0;
      return dropout_ws(sh, (int64_t)sh.B * n, n, n).total;
    case LISA_OP_LINEAR_UPDATE:
      return 256;  // no workspace is used; a nonzero size marks a valid shape
    default:
      fail(LISA_ERR_INVALID_ARG, "unknown op %d", op);
      return 0;
  }
}

int lisa_decode_step(const lisa_shape* shape, const int32_t* seq_lens, const void* q, const void* k_new,
                     const void* v_new, const void* q_idx, const void* k_idx_new, const void* q_lin,
                     const void* k_lin, const void* v_lin, const void* x, const void* w_gate,
                     const float* w_idx, void* k_cache, void* v_cache, void* k_idx_cache, float* S, float* z,
                     void* out, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_decode_len(sh))) return rc;
  return decode_step(sh, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin, x, w_gate, w_idx,
                     k_cache, v_cache, k_idx_cache, S, z, out, idx_out, ws, ws_bytes, stream);
}

int lisa_decode_step_noalloc(const lisa_shape* shape, const int32_t* seq_lens, const void* q, const void* k_new,
                             const void* v_new, const void* q_idx, const void* k_idx_new, const void* q_lin,
                             const void* k_lin, const void* v_lin, const void* x, const void* w_gate,
                             const float* w_idx, void* k_cache, void* v_cache, void* k_idx_cache, float* S,
                             float* z, void* out, int32_t* idx_out, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_decode_len(sh))) return rc;
  const size_t need = decode_ws(sh).total;
  if (need > LISA_DECODE_SCRATCH_BYTES)
    return fail(LISA_ERR_WORKSPACE,
                "this shape needs %zu bytes of decode workspace; the allocation-free decode step holds %zu "
                "(use lisa_decode_step with a caller workspace)",
                need, (size_t)LISA_DECODE_SCRATCH_BYTES);
  // every host-side check before the first HIP call
  if ((rc = decode_check_pointers(sh, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin, x, w_gate,
                                  w_idx, k_cache, v_cache, k_idx_cache, S, z, out, idx_out)))
    return rc;
  void* ws = nullptr;
  if ((rc = decode_scratch(ws))) return rc;
  return decode_step(sh, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin, x, w_gate, w_idx,
                     k_cache, v_cache, k_idx_cache, S, z, out, idx_out, ws, LISA_DECODE_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {

// The decode step's tensor arguments: present and 16-byte aligned (the
// indexer's only outside the sliding-window mode).
int decode_check_pointers(const Shape& sh, const int32_t* seq_lens, const void* q, const void* k_new,
                          const void* v_new, const void* q_idx, const void* k_idx_new, const void* q_lin,
                          const void* k_lin, const void* v_lin, const void* x, const void* w_gate,
                          const float* w_idx, void* k_cache, void* v_cache, void* k_idx_cache, float* S, float* z,
                          void* out, int32_t* idx_out) {
  REQUIRE_PTR(seq_lens); REQUIRE_PTR(q); REQUIRE_PTR(k_new); REQUIRE_PTR(v_new);
  REQUIRE_PTR(q_lin); REQUIRE_PTR(k_lin); REQUIRE_PTR(v_lin); REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache);
  REQUIRE_PTR(S); REQUIRE_PTR(z); REQUIRE_PTR(out); OPTIONAL_PTR(idx_out);
  if (!(sh.flags & LISA_SLIDING_WINDOW)) {
    REQUIRE_PTR(q_idx); REQUIRE_PTR(k_idx_new); REQUIRE_PTR(w_idx); REQUIRE_PTR(k_idx_cache);
  }
  return LISA_OK;
}

// The decode step after shape validation: pointer checks, then the launches
// on the workspace `ws` (caller-owned, or the static scratch).
int decode_step(const Shape& sh, const int32_t* seq_lens, const void* q, const void* k_new, const void* v_new,
                const void* q_idx, const void* k_idx_new, const void* q_lin, const void* k_lin, const void* v_lin,
                const void* x, const void* w_gate, const float* w_idx, void* k_cache, void* v_cache,
                void* k_idx_cache, float* S, float* z, void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                void* stream) {
  const bool window = sh.flags & LISA_SLIDING_WINDOW;  // no indexer: its arguments are not used
  // A budget of at least max_len keeps every position of every sequence, so
  // the scores cannot change the selection: the step appends the index key
  // but neither scores nor selects, and attends to positions 0 .. L-1 as the
  // window path does (a window of M >= L is the whole prefix).
  const bool take_all = !window && sh.M >= sh.max_len;
  int prc = decode_check_pointers(sh, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin, x, w_gate,
                                  w_idx, k_cache, v_cache, k_idx_cache, S, z, out, idx_out);
  if (prc) return prc;
  REQUIRE_PTR(ws);
  const DecodeWs w = decode_ws(sh);
  if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;

  PhaseAArgs pa{};
  pa.sh = sh;
  pa.seq_lens = seq_lens;
  pa.q_idx = q_idx; pa.k_idx_new = k_idx_new; pa.k_new = k_new; pa.v_new = v_new;
  pa.q_lin = q_lin; pa.k_lin = k_lin; pa.v_lin = v_lin; pa.x = x; pa.w_gate = w_gate; pa.w_idx = w_idx;
  pa.k_cache = k_cache; pa.v_cache = v_cache; pa.k_idx_cache = k_idx_cache; pa.S = S; pa.z = z;
  pa.scores = at<float>(ws, w.scores); pa.scores_ld = decode_scores_ld(sh);
  pa.o_lin = at<float>(ws, w.o_lin); pa.lin_den = at<float>(ws, w.lin_den);
  pa.gate_part = at<float>(ws, w.gate); pa.gate_chunks = decode_gate_chunks(sh);
  pa.append = 1; pa.do_scores = 1; pa.do_linear = 1; pa.do_gate = 1; pa.linear_output = 1;
  if (window || take_all) {  // append without scoring; the window's index list if asked for
    if (window) { pa.q_idx = nullptr; pa.k_idx_new = nullptr; pa.k_idx_cache = nullptr; pa.w_idx = nullptr; }
    pa.do_scores = 0; pa.window_idx = idx_out; pa.M = sh.M;
  }
  if (window || take_all) {
    LAUNCH(KID_DECODE_PHASE_A, st, launch_decode_phase_a(pa, st));
    AttnArgs aa{};
    aa.sh = sh; aa.n_rows = sh.B; aa.rows_per_seq = 1; aa.prefill = 0; aa.dense = 0; aa.window = 1;
    aa.seq_lens = seq_lens; aa.q = q; aa.k_cache = k_cache; aa.v_cache = v_cache; aa.idx = nullptr; aa.idx_ld = 0;
    aa.nsplit = w.nsplit; aa.split_len = w.split_len; aa.part = at<float>(ws, w.part);
    aa.gate_part = pa.gate_part; aa.gate_chunks = pa.gate_chunks;
    aa.o_lin = pa.o_lin; aa.lin_den = (sh.flags & LISA_LINEAR_UNNORMALIZED) ? nullptr : pa.lin_den; aa.out = out;
    LAUNCH(KID_ATTN, st, launch_attention(aa, st));
    LAUNCH(KID_ATTN_COMBINE, st, launch_attention_combine(aa, st));
    return LISA_OK;
  }

  LAUNCH(KID_DECODE_PHASE_A, st, launch_decode_phase_a(pa, st));
  const bool fused = decode_fused(sh, w.nsplit, w.split_len);
  int32_t* idx = idx_out ? idx_out : (fused ? nullptr : at<int32_t>(ws, w.idx));
  SelectArgs sa{};
  sa.n_rows = sh.B; sa.rows_per_seq = 1; sa.prefill = 0; sa.seq_lens = seq_lens;
  sa.scores = pa.scores; sa.ld = pa.scores_ld; sa.first_row = 0; sa.stored_rows = 1;
  sa.M = sh.M; sa.max_len = sh.max_len; sa.idx = idx; sa.idx_ld = sh.M; sa.mask = nullptr;

  AttnArgs aa{};
  aa.sh = sh; aa.n_rows = sh.B; aa.rows_per_seq = 1; aa.prefill = 0; aa.dense = 0; aa.seq_lens = seq_lens;
  aa.q = q; aa.k_cache = k_cache; aa.v_cache = v_cache; aa.idx = idx; aa.idx_ld = sh.M;
  aa.nsplit = w.nsplit; aa.split_len = w.split_len; aa.part = at<float>(ws, w.part);
  aa.gate_part = pa.gate_part; aa.gate_chunks = pa.gate_chunks;
  aa.o_lin = pa.o_lin; aa.lin_den = (sh.flags & LISA_LINEAR_UNNORMALIZED) ? nullptr : pa.lin_den; aa.out = out;
  if (fused) {
    LAUNCH(KID_SELECT_ATTN, st, launch_select_attend(aa, sa, st));
  } else {
    LAUNCH(KID_SELECT, st, launch_select(sa, st));
    LAUNCH(KID_ATTN, st, launch_attention(aa, st));
  }
  LAUNCH(KID_ATTN_COMBINE, st, launch_attention_combine(aa, st));
  return LISA_OK;
}

}  // namespace

extern "C" {

int lisa_dense_decode(const lisa_shape* shape, const int32_t* seq_lens, const void* q, const void* k_cache,
                      const void* v_cache, void* out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_decode_len(sh))) return rc;
  REQUIRE_PTR(seq_lens); REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(out);
  REQUIRE_PTR(ws);
  const DenseWs w = dense_ws(sh);
  if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  AttnArgs aa{};
  aa.sh = sh; aa.n_rows = sh.B; aa.rows_per_seq = 1; aa.prefill = 0; aa.dense = 1; aa.seq_lens = seq_lens;
  aa.q = q; aa.k_cache = k_cache; aa.v_cache = v_cache; aa.idx = nullptr; aa.idx_ld = 0;
  aa.nsplit = w.nsplit; aa.split_len = w.split_len; aa.part = at<float>(ws, w.part);
  aa.gate_part = nullptr; aa.gate_chunks = 0; aa.o_lin = nullptr; aa.lin_den = nullptr;
  aa.out = out;
  LAUNCH(KID_ATTN, st, launch_attention(aa, st));
  LAUNCH(KID_ATTN_COMBINE, st, launch_attention_combine(aa, st));
  return LISA_OK;
}

int lisa_indexer_topk(const lisa_shape* shape, int rows_mode, int32_t n, const int32_t* seq_lens,
                      const void* q_idx, const void* k_idx_cache, const float* w_idx, const float* scores_in,
                      int64_t scores_ld, float* scores_out, int32_t* idx_out, void* ws, size_t ws_bytes,
                      void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if (rows_mode != LISA_ROWS_DECODE && rows_mode != LISA_ROWS_PREFILL)
    return fail(LISA_ERR_INVALID_ARG, "rows_mode %d", rows_mode);
  if (sh.flags & LISA_SLIDING_WINDOW) return fail(LISA_ERR_INVALID_ARG, "a sliding-window shape has no indexer");
  const bool dec = rows_mode == LISA_ROWS_DECODE;
  if (dec) {
    if ((rc = check_decode_len(sh))) return rc;
    REQUIRE_PTR(seq_lens);
  } else if ((rc = check_prefill_len(sh, n))) {
    return rc;
  }
  const int longest = dec ? sh.max_len : n;
  REQUIRE_PTR(idx_out);
  OPTIONAL_PTR(scores_in);
  OPTIONAL_PTR(scores_out);
  if ((scores_in || scores_out) && (scores_ld < longest || scores_ld % 4))
    return fail(LISA_ERR_INVALID_ARG, "scores_ld %lld must be a multiple of 4 and >= the longest row %d",
                (long long)scores_ld, longest);
  if (!scores_in) {
    REQUIRE_PTR(q_idx); REQUIRE_PTR(k_idx_cache); REQUIRE_PTR(w_idx);
  }
  const TopkWs w = topk_ws(sh, rows_mode, n);
  if (!scores_in && !scores_out) {
    REQUIRE_PTR(ws);
    if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  }
  hipStream_t st = (hipStream_t)stream;

  SelectArgs sa{};
  sa.M = sh.M; sa.idx = idx_out; sa.idx_ld = sh.M; sa.mask = nullptr; sa.max_len = longest;
  if (dec) {
    sa.n_rows = sh.B; sa.rows_per_seq = 1; sa.prefill = 0; sa.seq_lens = seq_lens;
    sa.first_row = 0; sa.stored_rows = 1;
    if (scores_in) {
      sa.scores = scores_in; sa.ld = scores_ld;
    } else {
      PhaseAArgs pa{};
      pa.sh = sh; pa.seq_lens = seq_lens; pa.q_idx = q_idx; pa.k_idx_new = nullptr; pa.w_idx = w_idx;
      pa.k_idx_cache = const_cast<void*>(k_idx_cache);
      pa.scores = scores_out ? scores_out : at<float>(ws, w.scores);
      pa.scores_ld = scores_out ? scores_ld : decode_scores_ld(sh);
      pa.do_scores = 1;
      LAUNCH(KID_DECODE_PHASE_A, st, launch_decode_phase_a(pa, st));
      sa.scores = pa.scores; sa.ld = pa.scores_ld;
    }
  } else {
    sa.n_rows = sh.B * n; sa.rows_per_seq = n; sa.prefill = 1; sa.seq_lens = nullptr;
    if (scores_in) {
      sa.scores = scores_in; sa.ld = scores_ld; sa.first_row = 0; sa.stored_rows = n;
    } else {
      IndexScoreArgs ia{};
      ia.sh = sh; ia.n = n; ia.q_idx = q_idx; ia.k_idx = k_idx_cache; ia.w_idx = w_idx;
      if (scores_out) {
        ia.row0 = 0; ia.stored_rows = n; ia.scores = scores_out; ia.ld = scores_ld;
      } else {
        ia.row0 = n > sh.M ? sh.M : n; ia.stored_rows = n > sh.M ? n - sh.M : 0;
        ia.scores = at<float>(ws, w.scores); ia.ld = prefill_scores_ld(n);
      }
      LAUNCH(KID_PREFILL_INDEX, st, index_mfma_supported(sh) ? launch_index_scores_mfma(ia, st)
                                                             : launch_index_scores(ia, st));
      sa.scores = ia.scores; sa.ld = ia.ld; sa.first_row = ia.row0; sa.stored_rows = ia.stored_rows;
    }
  }
  if (dec) {
    // the core the decode step of this shape selects with
    int nsplit, split_len;
    decode_step_split(sh, nsplit, split_len);
    if (decode_fused(sh, nsplit, split_len)) {
      LAUNCH(KID_SELECT, st, launch_select_runs(sa, st));
      return LISA_OK;
    }
  }
  LAUNCH(KID_SELECT, st, launch_select(sa, st));
  return LISA_OK;
}

int lisa_linear_state_update(const lisa_shape* shape, int32_t n_tokens, const void* k_lin, const void* v_lin,
                             float* S, float* z, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if (n_tokens < 1) return fail(LISA_ERR_INVALID_ARG, "n_tokens %d", n_tokens);
  REQUIRE_PTR(k_lin); REQUIRE_PTR(v_lin); REQUIRE_PTR(S); REQUIRE_PTR(z);
  hipStream_t st = (hipStream_t)stream;
  if (linear_mfma_supported(sh)) {
    LinearChunkArgs lc{};
    lc.sh = sh; lc.n = n_tokens; lc.k_lin = k_lin; lc.v_lin = v_lin; lc.S = S; lc.z = z;
    lc.nseg = 1; lc.seg_len = (n_tokens + 63) / 64 * 64; lc.in_place = 1;
    LAUNCH(KID_LINEAR_UPDATE, st, launch_linear_seg_sums(lc, st));
    return LISA_OK;
  }
  LinearArgs la{};
  la.sh = sh; la.n = n_tokens; la.q_lin = nullptr; la.k_lin = k_lin; la.v_lin = v_lin;
  la.S = S; la.z_in = z; la.z_out = z; la.o_lin = nullptr;  // without outputs only slice 0 touches z
  LAUNCH(KID_LINEAR_UPDATE, st, launch_linear_recurrent(la, st));
  return LISA_OK;
}

int lisa_segment_correct(const lisa_shape* shape, float* S, float* z, float* S_start, float* z_start,
                         float* mean_S, float* mean_z, int32_t t, float alpha, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if (t < 1) return fail(LISA_ERR_INVALID_ARG, "segment number %d (must be >= 1)", t);
  if (!(fabsf(alpha) < INFINITY)) return fail(LISA_ERR_INVALID_ARG, "alpha is not finite");
  REQUIRE_PTR(S); REQUIRE_PTR(z); REQUIRE_PTR(S_start); REQUIRE_PTR(z_start); REQUIRE_PTR(mean_S);
  REQUIRE_PTR(mean_z);
  if (sh.d % 4) return fail(LISA_ERR_UNSUPPORTED, "head dim %d is not a multiple of 4", sh.d);
  SegmentArgs a{};
  a.S = S; a.z = z; a.S_start = S_start; a.z_start = z_start; a.mean_S = mean_S; a.mean_z = mean_z;
  a.n_S = (size_t)sh.B * sh.H_L * sh.d * sh.d; a.n_z = (size_t)sh.B * sh.H_L * sh.d;
  a.t = t; a.alpha = alpha;
  LAUNCH(KID_SEGMENT, (hipStream_t)stream, launch_segment_correct(a, (hipStream_t)stream));
  return LISA_OK;
}

int lisa_attention_mass(const lisa_shape* shape, int32_t n_rows, const int32_t* row_seq, const int32_t* row_len,
                        const void* q, const void* k_cache, const int32_t* idx, float* mass, float* bound,
                        void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_decode_len(sh))) return rc;
  if (n_rows < 0 || n_rows > 65535) return fail(LISA_ERR_INVALID_ARG, "n_rows %d outside [0, 65535]", n_rows);
  if (n_rows == 0) return LISA_OK;
  OPTIONAL_PTR(row_seq); REQUIRE_PTR(row_len); REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(idx);
  REQUIRE_PTR(mass); OPTIONAL_PTR(bound); REQUIRE_PTR(ws);
  if ((size_t)n_rows * sh.H_q > 0x7fffffffu) return fail(LISA_ERR_UNSUPPORTED, "n_rows * H_q too large");
  const MassWs w = mass_ws(sh, n_rows);
  if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  MassArgs a{};
  a.sh = sh; a.n_rows = n_rows; a.row_seq = row_seq; a.row_len = row_len; a.q = q; a.k_cache = k_cache;
  a.idx = idx; a.scale = 1.f / sqrtf((float)sh.d);
  a.logits = at<float>(ws, w.logits); a.ld = mass_logits_ld(sh); a.lens = at<int32_t>(ws, w.lens);
  a.bidx = bound ? at<int32_t>(ws, w.bidx) : nullptr; a.mass = mass; a.bound = bound;
  a.part = at<float2>(ws, w.part); a.part_ld = mass_key_blocks(sh.max_len);
  LAUNCH(KID_MASS_LOGITS, st, launch_mass_logits(a, sh.max_len, st));
  if (bound) {
    SelectArgs sa{};
    sa.n_rows = n_rows * sh.H_q; sa.rows_per_seq = 1; sa.prefill = 0; sa.seq_lens = a.lens;
    sa.scores = a.logits; sa.ld = a.ld; sa.first_row = 0; sa.stored_rows = 1; sa.M = sh.M;
    sa.max_len = sh.max_len; sa.idx = at<int32_t>(ws, w.bidx); sa.idx_ld = sh.M; sa.mask = nullptr;
    LAUNCH(KID_MASS_SELECT, st, launch_select(sa, st));
  }
  LAUNCH(KID_MASS_REDUCE, st, launch_mass_reduce(a, st));
  return LISA_OK;
}

int lisa_candidate_dropout(const lisa_shape* shape, int rows_mode, int32_t n, const int32_t* seq_lens,
                           const float* scores, const float* u, int64_t scores_ld, int32_t n_cand, float p,
                           int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if (rows_mode != LISA_ROWS_DECODE && rows_mode != LISA_ROWS_PREFILL)
    return fail(LISA_ERR_INVALID_ARG, "rows_mode %d", rows_mode);
  const bool dec = rows_mode == LISA_ROWS_DECODE;
  if (dec) {
    if ((rc = check_decode_len(sh))) return rc;
    REQUIRE_PTR(seq_lens);
  } else if ((rc = check_prefill_len(sh, n))) {
    return rc;
  }
  const int longest = dec ? sh.max_len : n;
  if (n_cand < 1) return fail(LISA_ERR_INVALID_ARG, "n_cand %d (must be >= 1)", n_cand);
  if (!(p == p)) return fail(LISA_ERR_INVALID_ARG, "p is NaN");
  REQUIRE_PTR(scores); REQUIRE_PTR(u); REQUIRE_PTR(idx_out); REQUIRE_PTR(ws);
  if (scores_ld < longest || scores_ld % 4)
    return fail(LISA_ERR_INVALID_ARG, "scores_ld %lld must be a multiple of 4 and >= the longest row %d",
                (long long)scores_ld, longest);
  const int64_t rows = dec ? sh.B : (int64_t)sh.B * n;
  if (rows > 0x7fffffff) return fail(LISA_ERR_UNSUPPORTED, "too many rows");
  const int cmax = min(n_cand, longest);
  const DropoutWs w = dropout_ws(sh, rows, longest, cmax);
  if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  SelectArgs sa{};
  sa.n_rows = (int)rows; sa.rows_per_seq = dec ? 1 : n; sa.prefill = dec ? 0 : 1; sa.seq_lens = dec ? seq_lens : nullptr;
  sa.scores = scores; sa.ld = scores_ld; sa.first_row = 0; sa.stored_rows = dec ? 1 : n; sa.max_len = longest;
  sa.M = n_cand; sa.idx = nullptr; sa.idx_ld = 0;
  sa.mask = at<uint32_t>(ws, w.mask); sa.mask_ld = dropout_mask_ld(longest);
  LAUNCH(KID_SELECT, st, launch_select(sa, st));  // 1. candidates
  DropoutArgs da{};
  da.n_rows = (int)rows; da.rows_per_seq = sa.rows_per_seq; da.prefill = sa.prefill; da.seq_lens = sa.seq_lens;
  da.scores = scores; da.u = u; da.ld = scores_ld; da.p = p; da.mask = sa.mask; da.mask_ld = sa.mask_ld;
  da.cnt = at<int32_t>(ws, w.cnt); da.cscore = at<float>(ws, w.cscore); da.cpos = at<int32_t>(ws, w.cpos);
  da.cld = dropout_cld(cmax); da.idx2 = at<int32_t>(ws, w.idx2); da.M = sh.M; da.idx_out = idx_out;
  LAUNCH(KID_DROPOUT, st, launch_dropout_compact(da, st));  // 2. survivor rows
  SelectArgs sb{};  // 3. the M best of each survivor row (decode rows of length cnt)
  sb.n_rows = (int)rows; sb.rows_per_seq = 1; sb.prefill = 0; sb.seq_lens = da.cnt;
  sb.scores = da.cscore; sb.ld = da.cld; sb.first_row = 0; sb.stored_rows = 1; sb.max_len = cmax;
  sb.M = sh.M; sb.idx = at<int32_t>(ws, w.idx2); sb.idx_ld = sh.M; sb.mask = nullptr;
  LAUNCH(KID_SELECT, st, launch_select(sb, st));
  const hipError_t e = launch_dropout_gather(da, st);  // 4. positions
  if (e != hipSuccess) return fail_hip(e, "dropout_gather");
  return LISA_OK;
}

int lisa_indexer_kl(const lisa_shape* shape, int32_t n, const void* q, const void* k_cache, const void* q_idx,
                    const void* k_idx_cache, float* kl_out, float* loss_out, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_prefill_len(sh, n))) return rc;
  if (sh.flags & LISA_SLIDING_WINDOW) return fail(LISA_ERR_INVALID_ARG, "a sliding-window shape has no indexer");
  if (sh.H_q % sh.H_I)
    return fail(LISA_ERR_UNSUPPORTED, "H_q (%d) is not a multiple of H_I (%d): teacher heads cannot be grouped",
                sh.H_q, sh.H_I);
  REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(q_idx); REQUIRE_PTR(k_idx_cache); REQUIRE_PTR(kl_out);
  OPTIONAL_PTR(loss_out);
  if ((size_t)sh.B * n * sh.H_I > 0x7fffffffu) return fail(LISA_ERR_UNSUPPORTED, "B * n * H_I too large");
  if (sh.B > 65535) return fail(LISA_ERR_UNSUPPORTED, "B %d > 65535", sh.B);
  hipStream_t st = (hipStream_t)stream;
  KlArgs a{};
  a.sh = sh; a.n = n; a.q = q; a.k_cache = k_cache; a.q_idx = q_idx; a.k_idx = k_idx_cache;
  a.scale = 1.f / sqrtf((float)sh.d); a.kl = kl_out; a.loss = loss_out;
  LAUNCH(KID_INDEXER_KL, st, launch_indexer_kl(a, st));
  if (loss_out) {
    const hipError_t e = launch_indexer_kl_loss(a, st);
    if (e != hipSuccess) return fail_hip(e, "indexer_kl_loss");
  }
  return LISA_OK;
}

int lisa_prefill(const lisa_shape* shape, int32_t n, const void* q, const void* k_cache, const void* v_cache,
                 const void* k_idx_cache, const void* q_idx, const void* q_lin, const void* k_lin,
                 const void* v_lin, const void* x, const void* w_gate, const float* w_idx, float* S, float* z,
                 void* out, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(shape, sh);
  if (rc) return rc;
  if ((rc = check_prefill_len(sh, n))) return rc;
  const bool window = sh.flags & LISA_SLIDING_WINDOW;  // no indexer: its arguments are not used
  REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache);
  REQUIRE_PTR(q_lin); REQUIRE_PTR(k_lin); REQUIRE_PTR(v_lin); REQUIRE_PTR(x); REQUIRE_PTR(w_gate);
  REQUIRE_PTR(S); REQUIRE_PTR(z); REQUIRE_PTR(out); OPTIONAL_PTR(idx_out); REQUIRE_PTR(ws);
  if (!window) {
    REQUIRE_PTR(k_idx_cache); REQUIRE_PTR(q_idx); REQUIRE_PTR(w_idx);
  }
  const PrefillWs w = prefill_ws(sh, n);
  if (ws_bytes < w.total) return fail(LISA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  // the gate and the linear branch depend on neither the indexer nor the
  // select: with a side stream they run next to them (not while the timing
  // hook is armed, so that a timed kernel runs alone)
  SideStream* side = (window || timing_armed()) ? nullptr : side_stream(st);
  hipStream_t sst = st;
  if (side) {
    hipError_t e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return fail_hip(e, "prefill fork");
    sst = side->s;
  }

  GateArgs ga{};
  ga.sh = sh; ga.n_rows = sh.B * n; ga.x = x; ga.w_gate = w_gate; ga.gate_part = at<float>(ws, w.gate);
  if (gate_mfma_supported(sh)) {
    ga.w_t = at<bf16_t>(ws, w.w_t);
    LAUNCH(KID_PREFILL_GATE_PREP, sst, launch_gate_transpose(ga, sst));
    LAUNCH(KID_PREFILL_GATE, sst, launch_gate_mfma(ga, sst));
  } else {
    LAUNCH(KID_PREFILL_GATE, sst, launch_gate_logits(ga, sst));
  }

  float* o_lin = at<float>(ws, w.o_lin);
  if (linear_mfma_supported(sh)) {
    LinearChunkArgs lc{};
    lc.sh = sh; lc.n = n; lc.q_lin = q_lin; lc.k_lin = k_lin; lc.v_lin = v_lin; lc.S = S; lc.z = z;
    lc.seg_state = at<float>(ws, w.seg); lc.in_place = 0; lc.o_lin = o_lin;
    linear_segments(sh, n, lc.nseg, lc.seg_len);
    LAUNCH(KID_PREFILL_LIN_SUMS, sst, launch_linear_seg_sums(lc, sst));
    LAUNCH(KID_PREFILL_LIN_PREFIX, sst, launch_linear_seg_prefix(lc, sst));
    LAUNCH(KID_PREFILL_LINEAR, sst, launch_linear_chunks(lc, sst));
  } else {
    LinearArgs la{};
    la.sh = sh; la.n = n; la.q_lin = q_lin; la.k_lin = k_lin; la.v_lin = v_lin; la.S = S;
    la.z_in = z; la.z_out = at<float>(ws, w.z_tmp); la.o_lin = o_lin;
    LAUNCH(KID_PREFILL_LINEAR, sst, launch_linear_recurrent(la, sst));
    LAUNCH(KID_PREFILL_LINEAR, sst, launch_copy_f32(z, la.z_out, (size_t)sh.B * sh.H_L * sh.d, sst));
  }

  const bool mfma_attn = attn_mfma_supported(sh);
  if (window) {  // sliding window: no scores, no select; attention over each row's window
    if (idx_out) LAUNCH(KID_SELECT, st, launch_window_index(idx_out, sh.B, n, sh.M, st));
    if (mfma_attn) {
      AttnMaskArgs am{};
      am.sh = sh; am.n = n; am.q = q; am.k_cache = k_cache; am.v_cache = v_cache; am.mask = nullptr;
      am.mask_ld = 0; am.scale_log2e = 1.4426950408889634f / sqrtf((float)sh.d);
      am.gate_part = ga.gate_part; am.o_lin = o_lin; am.out = out; am.window = 1;
      LAUNCH(KID_PREFILL_ATTN, st, launch_attn_prefill_mfma(am, st));
      return LISA_OK;
    }
    AttnArgs aa{};
    aa.sh = sh; aa.n_rows = sh.B * n; aa.rows_per_seq = n; aa.prefill = 1; aa.dense = 0; aa.window = 1;
    aa.seq_lens = nullptr; aa.q = q; aa.k_cache = k_cache; aa.v_cache = v_cache; aa.idx = nullptr; aa.idx_ld = 0;
    aa.nsplit = 1; aa.split_len = sh.M; aa.part = nullptr;
    aa.gate_part = ga.gate_part; aa.gate_chunks = 1; aa.o_lin = o_lin; aa.lin_den = nullptr; aa.out = out;
    LAUNCH(KID_PREFILL_ATTN, st, launch_attention(aa, st));
    return LISA_OK;
  }

  IndexScoreArgs ia{};
  ia.sh = sh; ia.n = n; ia.q_idx = q_idx; ia.k_idx = k_idx_cache; ia.w_idx = w_idx;
  ia.row0 = n > sh.M ? sh.M : n; ia.stored_rows = n > sh.M ? n - sh.M : 0;
  ia.scores = at<float>(ws, w.scores); ia.ld = prefill_scores_ld(n);
  LAUNCH(KID_PREFILL_INDEX, st, index_mfma_supported(sh) ? launch_index_scores_mfma(ia, st)
                                                         : launch_index_scores(ia, st));

  int32_t* idx = idx_out ? idx_out : (mfma_attn ? nullptr : at<int32_t>(ws, w.idx));
  SelectArgs sa{};
  sa.n_rows = sh.B * n; sa.rows_per_seq = n; sa.prefill = 1; sa.seq_lens = nullptr;
  sa.scores = ia.scores; sa.ld = ia.ld; sa.first_row = ia.row0; sa.stored_rows = ia.stored_rows;
  sa.M = sh.M; sa.max_len = n; sa.idx = idx; sa.idx_ld = sh.M;
  sa.mask = mfma_attn ? at<uint32_t>(ws, w.mask) : nullptr; sa.mask_ld = attn_mask_ld(n);
  LAUNCH(KID_SELECT, st, launch_select(sa, st));
  uint32_t* occ = mfma_attn ? at<uint32_t>(ws, w.occ) : nullptr;
  if (occ) LAUNCH(KID_PREFILL_OCCUPANCY, st, launch_mask_occupancy(sa.mask, sa.mask_ld, sh.B, n, occ, prefill_occ_ld(n), st));
  if (side) {  // join: the attention reads the gate logits and the linear outputs
    hipError_t e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
    if (e != hipSuccess) return fail_hip(e, "prefill join");
  }

  if (mfma_attn) {
    AttnMaskArgs am{};
    am.sh = sh; am.n = n; am.q = q; am.k_cache = k_cache; am.v_cache = v_cache; am.mask = sa.mask;
    am.mask_ld = sa.mask_ld; am.scale_log2e = 1.4426950408889634f / sqrtf((float)sh.d);
    am.gate_part = ga.gate_part; am.o_lin = o_lin; am.out = out; am.occ = occ; am.occ_ld = prefill_occ_ld(n);
    LAUNCH(KID_PREFILL_ATTN, st, launch_attn_prefill_mfma(am, st));
    return LISA_OK;
  }
  AttnArgs aa{};
  aa.sh = sh; aa.n_rows = sh.B * n; aa.rows_per_seq = n; aa.prefill = 1; aa.dense = 0; aa.seq_lens = nullptr;
  aa.q = q; aa.k_cache = k_cache; aa.v_cache = v_cache; aa.idx = idx; aa.idx_ld = sh.M;
  aa.nsplit = 1; aa.split_len = sh.M; aa.part = nullptr;
  aa.gate_part = ga.gate_part; aa.gate_chunks = 1; aa.o_lin = o_lin; aa.lin_den = nullptr; aa.out = out;
  LAUNCH(KID_PREFILL_ATTN, st, launch_attention(aa, st));
  return LISA_OK;
}

}  // extern "C"
