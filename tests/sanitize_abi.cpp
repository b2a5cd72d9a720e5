// sanitize_abi.cpp -- drives the host-side argument validation of every
// libspecverify entry point (sizes, settings, null pointers, misaligned
// data and workspace, dtypes, strides, pools, processors, outcome sets) and
// the pure host queries (workspace sizes, path choice, status strings), in a
// build of the library whose host code runs under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every call checked here returns before any
// kernel is launched.  Test infrastructure: built and run by
// tests/test_sanitizers.py.  Exits 0 when every call returned the status its
// arguments call for.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "specverify.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAILED: %s: got %d, want %d\n", what, got, want);
    failures++;
  }
}

int main() {
  alignas(256) static unsigned char ws[1 << 16];
  const spec_sampling_t ok = {1.0f, 0, 0.95f}, plain = {1.0f, 0, 1.0f};
  const spec_sampling_t bad_t = {0.0f, 0, 1.0f}, bad_k = {1.0f, -1, 1.0f}, bad_p = {1.0f, 0, 1.5f};
  const int32_t V = 1000, k = 4, B = 3;
  // fake device addresses: validation never dereferences them
  const uintptr_t base = 1u << 20;
  spec_logits_t t = {reinterpret_cast<const void*>(base), SPEC_DTYPE_BF16, 0, (k + 1) * V, V};
  spec_logits_t d = {reinterpret_cast<const void*>(base), SPEC_DTYPE_BF16, 0, k * V, V};
  auto* i32 = reinterpret_cast<int32_t*>(base);
  auto* f32 = reinterpret_cast<float*>(base);

  // workspace sizes
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, B, k, V, &ok) > 0, 1, "size stochastic");
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, 0, k, V, &ok) == 0, 1, "size B = 0");
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, B, SPEC_MAX_K + 1, V, &ok) == 0, 1, "size k");
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, B, k, SPEC_MAX_V + 1, &ok) == 0, 1, "size V");
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, B, k, V, &bad_t) == 0, 1, "size T");
  expect(spec_workspace_size(SPEC_OP_STOCHASTIC, B, k, V, nullptr) == 0, 1, "size null sampling");
  expect(spec_workspace_size(SPEC_OP_GREEDY, B, k, V, nullptr) > 0, 1, "size greedy");
  expect(spec_workspace_size(SPEC_OP_PROCESS, 17, 0, V, &ok) > 0, 1, "size process");
  expect(spec_workspace_size(SPEC_OP_GREEDY_LMHEAD, B, k, V, nullptr) > 0, 1, "size lmhead");
  expect(spec_workspace_size(99, B, k, V, &ok) == 0, 1, "size bad op");
  expect(spec_workspace_size_pooled(SPEC_OP_STOCHASTIC, 10, 8, B, k, V, &ok) > 0, 1, "size pooled");
  expect(spec_workspace_size_pooled(SPEC_OP_GREEDY, 0, 0, B, k, V, nullptr) == 0, 1,
         "size pooled empty");

  // stochastic verify
  const size_t wsz = sizeof ws;
  expect(spec_verify_stochastic(t, d, i32, f32, 0, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic B = 0");
  expect(spec_verify_stochastic(t, d, i32, f32, B, 0, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic k = 0");
  expect(spec_verify_stochastic(t, d, i32, f32, B, 65, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_UNSUPPORTED, "stochastic k = 65");
  expect(spec_verify_stochastic(t, d, i32, f32, B, k, V, &bad_k, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic top_k < 0");
  expect(spec_verify_stochastic(t, d, i32, f32, B, k, V, &bad_p, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic top_p > 1");
  expect(spec_verify_stochastic(t, d, nullptr, f32, B, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic null tokens");
  expect(spec_verify_stochastic(t, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, nullptr, wsz, nullptr),
         SPEC_ERR_WORKSPACE, "stochastic null workspace");
  expect(spec_verify_stochastic(t, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws + 1, wsz - 1,
                                nullptr),
         SPEC_ERR_WORKSPACE, "stochastic misaligned workspace");
  expect(spec_verify_stochastic(t, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws, 16, nullptr),
         SPEC_ERR_WORKSPACE, "stochastic small workspace");
  spec_logits_t tf = t;
  tf.dtype = SPEC_DTYPE_F32;
  expect(spec_verify_stochastic(tf, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic dtype mismatch");
  spec_logits_t tx = t;
  tx.dtype = 7;
  expect(spec_verify_stochastic(tx, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_UNSUPPORTED, "stochastic unknown dtype");
  spec_logits_t ts = t;
  ts.pos_stride = V - 1;
  expect(spec_verify_stochastic(ts, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic short rows");
  spec_logits_t tm = t;
  tm.data = reinterpret_cast<const void*>(base + 1);
  expect(spec_verify_stochastic(tm, d, i32, f32, B, k, V, &ok, i32, i32, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "stochastic misaligned logits");

  // greedy and processing
  expect(spec_verify_greedy(t, i32, B, k, V, nullptr, i32, ws, wsz, nullptr), SPEC_ERR_INVALID_ARG,
         "greedy null output");
  expect(spec_verify_greedy(t, i32, B, k, V, i32, i32, ws, 8, nullptr), SPEC_ERR_WORKSPACE,
         "greedy small workspace");
  expect(spec_logits_process(t, 0, V, &ok, nullptr, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "process R = 0");
  expect(spec_logits_process(t, 5, V, &bad_t, nullptr, nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "process T = 0");

  // pooled rows
  expect(spec_verify_stochastic_pooled(t, 0, i32, d, 4, i32, i32, f32, B, k, V, &ok, i32, i32,
                                       nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "pooled empty target pool");
  expect(spec_verify_stochastic_pooled(t, 2, nullptr, d, 4, i32, i32, f32, B, k, V, &ok, i32, i32,
                                       nullptr, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "pooled default map, pool too small");
  expect(spec_verify_greedy_pooled(t, 1, nullptr, i32, B, k, V, i32, i32, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "greedy pooled pool too small");

  // fused LM head
  const void* h = reinterpret_cast<const void*>(base);
  expect(spec_verify_greedy_lmhead(h, 5 * 64, 64, h, 64, 48, i32, B, k, V, i32, i32, ws, wsz,
                                   nullptr),
         SPEC_ERR_INVALID_ARG, "lmhead d not a multiple of 32");
  expect(spec_verify_greedy_lmhead(h, 5 * 128, 128, h, 64, 128, i32, B, k, V, i32, i32, ws,
                                   wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "lmhead weight stride below d");
  expect(spec_verify_greedy_lmhead(h, 5 * 64, 64, h, 1 << 17, 1 << 17, i32, B, k, V, i32, i32, ws,
                                   wsz, nullptr),
         SPEC_ERR_UNSUPPORTED, "lmhead d above 65536");
  expect(spec_verify_greedy_lmhead(h, 5 * 64, 64, reinterpret_cast<const void*>(base + 8), 64, 64,
                                   i32, B, k, V, i32, i32, ws, wsz, nullptr),
         SPEC_ERR_INVALID_ARG, "lmhead misaligned weight");

  // processors and outcome lookup
  spec_processors_t proc = {nullptr, 0, 0, nullptr, 0, 0, 0.0f};
  expect(spec_logits_apply(t, B, k + 1, V, &proc, t, nullptr), SPEC_ERR_INVALID_ARG,
         "apply theta = 0");
  proc.theta = 1.2f;
  expect(spec_logits_apply(t, B, 2 * SPEC_MAX_K + 2, V, &proc, t, nullptr), SPEC_ERR_UNSUPPORTED,
         "apply too many rows");
  expect(spec_logits_apply(t, B, k + 1, V, nullptr, t, nullptr), SPEC_ERR_INVALID_ARG,
         "apply null processors");
  expect(spec_outcome_lookup(i32, i32, B, k, i32, i32, 0, i32, nullptr, nullptr),
         SPEC_ERR_INVALID_ARG, "lookup P = 0");
  expect(spec_outcome_lookup(i32, i32, B, k, i32, i32, 4097, i32, nullptr, nullptr),
         SPEC_ERR_UNSUPPORTED, "lookup P too large");

  // host queries
  const int cus = spec_device_cu_count(nullptr);
  expect(cus > 0, 1, "cu count");
  t.seq_stride = (k + 1) * 151936;
  t.pos_stride = 151936;
  d.seq_stride = k * 151936;
  d.pos_stride = 151936;
  expect(spec_verify_stochastic_path(t, d, 2 * cus, k, 151936, &ok, 0, nullptr),
         SPEC_PATH_TASK_QUEUE, "path task queue");
  expect(spec_verify_stochastic_path(t, d, 2 * cus, k, 151936, &ok, 1, nullptr),
         SPEC_PATH_SEQUENCE_WALK, "path walk");
  expect(spec_verify_stochastic_path(t, d, 2 * cus - 1, k, 151936, &plain, 0, nullptr),
         SPEC_PATH_ROW_PASS, "path row pass");
  expect(spec_verify_stochastic_path(t, d, 0, k, 151936, &ok, 0, nullptr), -SPEC_ERR_INVALID_ARG,
         "path B = 0");
  for (int s = -1; s < 7; ++s) {
    const char* msg = spec_status_string(s);
    expect(msg != nullptr && std::strlen(msg) > 0, 1, "status string");
  }
  if (failures) return 1;
  std::printf("sanitized host validation ok\n");
  return 0;
}
