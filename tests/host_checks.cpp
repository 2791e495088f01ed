// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; no GPU is needed and no kernel
// is launched).  Every call here must be rejected or answered on the host
// before any HIP call; the sanitizers report any out-of-bounds access,
// overflow or other undefined behaviour on those paths.  Built and run by
// tests/test_host_sanitizers.py; exits 0 when every expectation holds.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "lisa.h"

static int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, \
                  lisa_last_error());                                      \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static lisa_shape qwen7b() {
  lisa_shape s;
  std::memset(&s, 0, sizeof(s));
  s.B = 1; s.H_q = 28; s.H_kv = 4; s.d = 128; s.H_I = 4; s.H_Ik = 4; s.d_I = 64; s.H_L = 28;
  s.hidden = 3584; s.M = 2048; s.cap = 16384; s.max_len = 16384; s.chunk = 64; s.dtype = LISA_BF16;
  return s;
}

int main() {
  alignas(16) static unsigned char buf[4096];
  void* p = buf;                   // a valid, aligned host address (never dereferenced by the calls below)
  void* mis = buf + 8;             // misaligned
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  float* fp = reinterpret_cast<float*>(buf);

  // workspace sizes over every op, lengths at and past the limits, and shape
  // fields at extreme values
  lisa_shape s = qwen7b();
  const int ops[] = {LISA_OP_DECODE, LISA_OP_PREFILL, LISA_OP_TOPK_DECODE, LISA_OP_TOPK_PREFILL, LISA_OP_DENSE_DECODE,
                     LISA_OP_LINEAR_UPDATE, LISA_OP_MASS, LISA_OP_DROPOUT_DECODE, LISA_OP_DROPOUT_PREFILL, -1, 99};
  const int32_t ns[] = {INT_MIN, -1, 0, 1, 63, 64, 65, 2048, 16384, 65536, 65537, INT_MAX};
  for (int op : ops)
    for (int32_t n : ns) (void)lisa_workspace_bytes(&s, op, n);
  EXPECT(lisa_workspace_bytes(&s, LISA_OP_DECODE, 0) > 0);
  EXPECT(lisa_workspace_bytes(&s, LISA_OP_PREFILL, 16384) > 0);
  EXPECT(lisa_workspace_bytes(&s, LISA_OP_PREFILL, 65537) == 0);
  EXPECT(lisa_workspace_bytes(&s, 99, 0) == 0);
  EXPECT(lisa_workspace_bytes(nullptr, LISA_OP_DECODE, 0) == 0);
  const int32_t extremes[] = {INT_MIN, -1, 0, 1, 3, 7, 1 << 20, INT_MAX};
  for (int field = 0; field < 14; ++field)
    for (int32_t v : extremes) {
      lisa_shape t = qwen7b();
      reinterpret_cast<int32_t*>(&t)[field] = v;
      for (int op : ops) (void)lisa_workspace_bytes(&t, op, 4096);
    }
  lisa_shape flagged = qwen7b();
  flagged.flags = 0xffffffffu;
  (void)lisa_workspace_bytes(&flagged, LISA_OP_DECODE, 0);
  lisa_shape big = qwen7b();
  big.B = INT_MAX;
  EXPECT(lisa_workspace_bytes(&big, LISA_OP_DECODE, 0) == 0 || lisa_workspace_bytes(&big, LISA_OP_DECODE, 0) > (size_t)1 << 40);

  // status strings, kernel names, the timing hook's argument checks
  for (int c = -10; c <= 10; ++c) EXPECT(lisa_status_string(c) != nullptr);
  for (int k = -5; k < 40; ++k) (void)lisa_kernel_name(k);
  EXPECT(lisa_kernel_name(0) != nullptr && lisa_kernel_name(-1) == nullptr && lisa_kernel_name(1000) == nullptr);
  EXPECT(lisa_timing_enable(-3, nullptr, nullptr, 4) != 0);
  EXPECT(lisa_timing_enable(1000, nullptr, nullptr, 4) != 0);
  EXPECT(lisa_timing_count() == 0);

  // entry points with a NULL, a misaligned pointer or a bad argument: a
  // status code, no HIP call
  EXPECT(lisa_decode_step(&s, ip, nullptr, p, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr, p,
                          (size_t)1 << 40, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_decode_step(&s, ip, p, mis, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr, p,
                          (size_t)1 << 40, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_decode_step(&s, ip, p, p, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr, p, 100, nullptr) ==
         LISA_ERR_WORKSPACE);
  EXPECT(lisa_decode_step(nullptr, ip, p, p, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr, p,
                          (size_t)1 << 40, nullptr) != LISA_OK);
  EXPECT(lisa_decode_step_noalloc(&s, ip, nullptr, p, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr,
                                  nullptr) == LISA_ERR_INVALID_ARG);
  lisa_shape huge = qwen7b();
  huge.B = 64;
  EXPECT(lisa_decode_step_noalloc(&huge, ip, p, p, p, p, p, p, p, p, p, p, fp, p, p, p, fp, fp, p, nullptr,
                                  nullptr) == LISA_ERR_WORKSPACE);
  for (int32_t n : {INT_MIN, -1, 0, 65537, INT_MAX})
    EXPECT(lisa_prefill(&s, n, p, p, p, p, p, p, p, p, p, p, fp, fp, fp, p, nullptr, p, (size_t)1 << 40, nullptr) ==
           LISA_ERR_INVALID_ARG);
  EXPECT(lisa_prefill(&s, 100, p, p, p, p, p, p, p, p, p, p, fp, fp, fp, p, nullptr, p, 16, nullptr) ==
         LISA_ERR_WORKSPACE);
  EXPECT(lisa_indexer_topk(&s, 7, 10, ip, p, p, fp, nullptr, 0, nullptr, (int32_t*)p, p, (size_t)1 << 40, nullptr) ==
         LISA_ERR_INVALID_ARG);
  EXPECT(lisa_indexer_topk(&s, LISA_ROWS_DECODE, 0, ip, p, p, fp, fp, 100, nullptr, (int32_t*)p, p, (size_t)1 << 40,
                           nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_indexer_topk(&s, LISA_ROWS_DECODE, 0, ip, p, p, fp, fp, -4, nullptr, (int32_t*)p, p, (size_t)1 << 40,
                           nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_linear_state_update(&s, 0, p, p, fp, fp, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_linear_state_update(&s, -5, p, p, fp, fp, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_segment_correct(&s, fp, fp, fp, fp, fp, fp, 0, 0.5f, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_segment_correct(&s, fp, fp, fp, fp, fp, fp, 1, -1.0f / 0.0f, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_dense_decode(&s, ip, nullptr, p, p, p, p, (size_t)1 << 40, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_attention_mass(&s, -1, nullptr, ip, p, p, ip, fp, nullptr, p, (size_t)1 << 40, nullptr) ==
         LISA_ERR_INVALID_ARG);
  EXPECT(lisa_attention_mass(&s, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                             nullptr) == LISA_OK);
  EXPECT(lisa_indexer_kl(&s, 0, p, p, p, p, fp, nullptr, nullptr) == LISA_ERR_INVALID_ARG);
  EXPECT(lisa_indexer_kl(&s, 64, p, p, p, p, nullptr, nullptr, nullptr) == LISA_ERR_INVALID_ARG);
  int32_t* op = reinterpret_cast<int32_t*>(buf);
  EXPECT(lisa_candidate_dropout(&s, 0, 0, ip, fp, fp, 16384, 0, 0.2f, op, p, (size_t)1 << 40, nullptr) ==
         LISA_ERR_INVALID_ARG);
  EXPECT(lisa_candidate_dropout(&s, 9, 0, ip, fp, fp, 16384, 2458, 0.2f, op, p, (size_t)1 << 40, nullptr) ==
         LISA_ERR_INVALID_ARG);
  EXPECT(std::strlen(lisa_last_error()) > 0);

  std::printf("%s: %d failures\n", failures ? "host checks FAILED" : "host checks passed", failures);
  return failures ? 1 : 0;
}
