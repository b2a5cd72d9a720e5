/*
 * sanitize_oracle.c -- drives every entry point of the CPU oracle (oracle.c)
 * over small synthetic inputs so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check its memory accesses and arithmetic:
 * fp32 and bf16 rows, temperature, top-k (ties, k >= V), top-p, -inf
 * masks, NaN / +inf rows, out-of-range tokens, V = 1, k up to 8, broadcast
 * sequences (stride 0).  Test infrastructure: built and run by
 * tests/test_sanitizers.py on the host.  Exits 0 when every call returned
 * the status its inputs call for.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform01(void) { /* xorshift64*, enough for test inputs */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static float normal(float sigma) {
  double u1 = uniform01(), u2 = uniform01();
  if (u1 < 1e-300) u1 = 1e-300;
  return (float)(sigma * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static uint16_t to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    failures++;
  }
}

static void run_case(int B, int k, int V, int bf16, double T, int top_k, double top_p,
                     int mask, int poison) {
  const int nt = B * (k + 1) * V, nd = B * k * V;
  float* tf = (float*)malloc(sizeof(float) * (size_t)nt);
  float* df = (float*)malloc(sizeof(float) * (size_t)nd);
  uint16_t* tb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nt);
  uint16_t* db = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nd);
  int* tokens = (int*)malloc(sizeof(int) * (size_t)(B * k));
  float* u = (float*)malloc(sizeof(float) * (size_t)(B * (k + 1)));
  int* acc = (int*)malloc(sizeof(int) * (size_t)B);
  int* out = (int*)malloc(sizeof(int) * (size_t)(B * (k + 1)));
  double* ap = (double*)malloc(sizeof(double) * (size_t)(B * k));
  int* flags = (int*)malloc(sizeof(int) * (size_t)B);
  double* prob = (double*)malloc(sizeof(double) * (size_t)V);
  double stats[5];
  for (int i = 0; i < nt; i++) tf[i] = normal(2.0f);
  for (int b = 0; b < B; b++)
    for (int j = 0; j < k; j++)
      for (int x = 0; x < V; x++)
        df[(b * k + j) * V + x] = tf[(b * (k + 1) + j) * V + x] + normal(0.7f);
  if (mask)
    for (int i = 0; i < nt; i++)
      if (uniform01() < 0.3 && i % V != 0) tf[i] = -INFINITY;
  if (poison && nt > 3) {
    tf[1] = NAN;      /* sequence 0, target row 0 */
    df[nd - 1] = INFINITY;
  }
  for (int i = 0; i < nt; i++) tb[i] = to_bf16(tf[i]);
  for (int i = 0; i < nd; i++) db[i] = to_bf16(df[i]);
  const void* T_ = bf16 ? (const void*)tb : (const void*)tf;
  const void* D_ = bf16 ? (const void*)db : (const void*)df;
  const int dt = bf16 ? ORC_BF16 : ORC_F32;
  for (int b = 0; b < B; b++)
    for (int j = 0; j < k; j++) {
      const int r = orc_sample_row((const char*)D_ + (size_t)((b * k + j) * V) * (bf16 ? 2 : 4), dt,
                                   V, T, top_k, top_p, uniform01());
      tokens[b * k + j] = r >= 0 ? r : 0;
    }
  if (poison) tokens[0] = V; /* out of range */
  for (int i = 0; i < B * (k + 1); i++) u[i] = (float)uniform01();
  int rc = orc_verify_stochastic(T_, (long long)(k + 1) * V, V, D_, (long long)k * V, V, dt,
                                 tokens, u, B, k, V, T, top_k, top_p, acc, out, ap, flags);
  expect(rc == 0, "orc_verify_stochastic returns 0");
  for (int b = 0; b < B; b++) {
    expect(acc[b] >= -1 && acc[b] <= k, "accepted length in range");
    if (acc[b] >= 0) expect(out[b * (k + 1) + acc[b]] >= 0 && out[b * (k + 1) + acc[b]] < V,
                            "emitted token in range");
  }
  /* broadcast target (sequence stride 0) */
  rc = orc_verify_stochastic(T_, 0, V, D_, (long long)k * V, V, dt, tokens, u, B, k, V, T, top_k,
                             top_p, acc, out, NULL, NULL);
  expect(rc == 0, "broadcast verify returns 0");
  rc = orc_verify_greedy(T_, (long long)(k + 1) * V, V, dt, tokens, B, k, V, acc, out);
  expect(rc == 0, "orc_verify_greedy returns 0");
  for (int r = 0; r < B * (k + 1); r++) {
    const void* row = (const char*)T_ + (size_t)(r * V) * (bf16 ? 2 : 4);
    const int ok = orc_process_row(row, dt, V, T, top_k, top_p, prob, stats);
    if (ok) {
      double s = 0.0;
      for (int x = 0; x < V; x++) s += prob[x];
      expect(fabs(s - 1.0) < 1e-9, "processed row sums to one");
    }
    (void)orc_process_row(row, dt, V, T, top_k, top_p, NULL, NULL);
    (void)orc_argmax_row(row, dt, V);
  }
  free(tf), free(df), free(tb), free(db), free(tokens), free(u), free(acc), free(out), free(ap);
  free(flags), free(prob);
}

int main(void) {
  run_case(3, 4, 257, 0, 1.0, 0, 1.0, 0, 0);
  run_case(3, 4, 257, 1, 0.7, 0, 0.95, 0, 0);
  run_case(2, 3, 100, 1, 1.0, 5, 0.9, 1, 0);
  run_case(2, 3, 100, 0, 1.3, 100, 0.5, 1, 0);
  run_case(2, 3, 100, 0, 1.0, 250, 1.0, 0, 1);
  run_case(4, 1, 1, 0, 1.0, 0, 1.0, 0, 0);
  run_case(1, 8, 33, 1, 0.5, 1, 0.3, 0, 1);
  run_case(5, 2, 7, 1, 2.0, 3, 0.99, 1, 0);
  if (failures) return 1;
  printf("sanitized oracle run ok\n");
  return 0;
}
