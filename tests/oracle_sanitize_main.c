/* Test driver (CPU): runs every oracle function on small seeded random layers so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer checks the oracle's memory
 * accesses and arithmetic (out-of-bounds reads and writes, leaks, signed overflow, bad
 * shifts). Sizes include empty batches, a single expert, k = E, padded and ragged buffers,
 * drops, every dtype and activation. Also checks that the expert-grouped path (rows,
 * then combine) and the per-token path (layer_tokens) agree. Prints "ok" on success. */
#include "../oracle/moe_oracle.c"

#include <stdio.h>

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static double urand(void) {  /* xorshift64, uniform in [0, 1) */
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}
static int irand(int lo, int hi) { return lo + (int)(urand() * (double)(hi - lo + 1)); }
static double nrand(void) { return 2.0 * urand() - 1.0; }
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}
static void* xalloc(size_t n) {  /* at least one byte, zeroed */
  void* p = calloc(n > 0 ? n : 1, 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}
/* fills an array of n elements of dtype 0 (fp32), 1 (bf16) or 2 (int8) */
static void* rand_array(int64_t n, int dtype, double scale) {
  const size_t es = dtype == 0 ? 4 : (dtype == 1 ? 2 : 1);
  void* p = xalloc((size_t)n * es);
  for (int64_t i = 0; i < n; ++i) {
    const float v = (float)(scale * nrand());
    if (dtype == 0) ((float*)p)[i] = v;
    else if (dtype == 1) ((uint16_t*)p)[i] = bf16_of(v);
    else ((int8_t*)p)[i] = (int8_t)irand(-127, 127);
  }
  return p;
}
static float* rand_scales(int64_t n) {
  float* s = (float*)xalloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) s[i] = (float)(0.001 + 0.01 * urand());
  return s;
}

int main(void) {
  for (int it = 0; it < 80; ++it) {
    const int64_t N = it % 17 == 0 ? 0 : irand(1, 40);
    const int32_t E = it % 13 == 0 ? 1 : irand(1, 12);
    const int32_t k = it % 11 == 0 ? E : irand(1, E < 4 ? E : 4);
    const int64_t D = 8 * irand(1, 6), F = 8 * irand(1, 6);
    const int xdt = it % 2, wdt = it % 3, act = (it / 3) % 3, mode = (it / 2) % 2;
    const int noisy = (it / 5) % 3;
    void* x = rand_array(N * D, xdt, 1.0);
    float* w_r = (float*)rand_array(D * E, 0, 0.5);
    float* bias = it % 4 == 0 ? NULL : (float*)rand_array(E, 0, 1.0);
    float* noise = (float*)rand_array(N * E, 0, 1.0);
    double* logits = (double*)xalloc(sizeof(double) * (size_t)(N * E));
    oracle_router_logits(N, D, E, xdt, x, w_r, bias, logits);
    int32_t* idx = (int32_t*)xalloc(sizeof(int32_t) * (size_t)(N * k));
    double* gate = (double*)xalloc(sizeof(double) * (size_t)(N * k));
    double* probs = (double*)xalloc(sizeof(double) * (size_t)(N * E));
    double* margin = (double*)xalloc(sizeof(double) * (size_t)N);
    if (oracle_route(N, E, k, mode, noisy, logits, noisy ? noise : NULL, idx, gate, probs, margin) != ORACLE_OK) {
      fprintf(stderr, "route failed at %d\n", it);
      return 1;
    }
    int64_t C = -1;
    const int capped = it % 3 != 0;
    if (capped && oracle_capacity(N, E, k, 0.25 * irand(1, 6), irand(0, 3), it % 2, &C) != ORACLE_OK) {
      fprintf(stderr, "capacity failed at %d\n", it);
      return 1;
    }
    const int padded = capped && it % 2 == 1;
    int64_t* load = (int64_t*)xalloc(sizeof(int64_t) * (size_t)E);
    int64_t* counts = (int64_t*)xalloc(sizeof(int64_t) * (size_t)E);
    int64_t* offsets = (int64_t*)xalloc(sizeof(int64_t) * (size_t)(E + 1));
    int64_t* row_of = (int64_t*)xalloc(sizeof(int64_t) * (size_t)(N * k));
    uint8_t* dropped = (uint8_t*)xalloc((size_t)(N * k));
    if (oracle_dispatch(N, E, k, idx, C, padded, (it / 7) % 2, load, counts, offsets, row_of, dropped) != ORACLE_OK) {
      fprintf(stderr, "dispatch failed at %d\n", it);
      return 1;
    }
    double* gate_eff = (double*)xalloc(sizeof(double) * (size_t)(N * k));
    oracle_drop_rule(N, k, gate, dropped, gate_eff);
    /* expert-grouped path: the filled buffer rows, their expert outputs, the combine */
    const int64_t rows = offsets[E];
    double* xrows = (double*)xalloc(sizeof(double) * (size_t)(rows * D));
    int32_t* experts = (int32_t*)xalloc(sizeof(int32_t) * (size_t)rows);
    for (int64_t t = 0; t < N; ++t)
      for (int32_t j = 0; j < k; ++j) {
        const int64_t r = row_of[t * k + j];
        if (r < 0) continue;
        if (r >= rows) { fprintf(stderr, "row out of range at %d\n", it); return 1; }
        experts[r] = idx[t * k + j];
        for (int64_t d = 0; d < D; ++d) xrows[r * D + d] = elem(x, xdt, t * D + d);
      }
    void* w1 = rand_array(E * D * F, wdt, 0.2);
    void* w2 = rand_array(E * D * F, wdt, 0.2);
    void* w3 = rand_array(E * F * D, wdt, 0.2);
    float* s1 = wdt == W_INT8 ? rand_scales(E * F) : NULL;
    float* s2 = wdt == W_INT8 ? rand_scales(E * F) : NULL;
    float* s3 = wdt == W_INT8 ? rand_scales(E * D) : NULL;
    double* hid = (double*)xalloc(sizeof(double) * (size_t)(rows * F));
    double* y_perm = (double*)xalloc(sizeof(double) * (size_t)(rows * D));
    if (oracle_expert_rows(rows, D, F, wdt, act, xrows, experts, w1, s1, w2, s2, w3, s3, hid, y_perm) != ORACLE_OK) {
      fprintf(stderr, "expert rows failed at %d\n", it);
      return 1;
    }
    double* y = (double*)xalloc(sizeof(double) * (size_t)(N * D));
    oracle_combine(N, D, k, y_perm, row_of, gate_eff, y);
    /* per-token path */
    int64_t* toks = (int64_t*)xalloc(sizeof(int64_t) * (size_t)N);
    for (int64_t t = 0; t < N; ++t) toks[t] = t;
    double* y2 = (double*)xalloc(sizeof(double) * (size_t)(N * D));
    if (oracle_layer_tokens(N, toks, N, D, F, E, k, xdt, wdt, act, x, w1, s1, w2, s2, w3, s3, idx, dropped, gate_eff,
                            y2) != ORACLE_OK) {
      fprintf(stderr, "layer tokens failed at %d\n", it);
      return 1;
    }
    for (int64_t i = 0; i < N * D; ++i)
      if (fabs(y[i] - y2[i]) > 1e-12 * (1.0 + fabs(y2[i]))) {
        fprintf(stderr, "grouped and per-token outputs differ at %d\n", it);
        return 1;
      }
    if (N > 0) {
      double* P = (double*)xalloc(sizeof(double) * (size_t)E);
      double b, bn;
      oracle_balance(N, E, k, probs, load, P, &b, &bn);
      free(P);
    }
    free(x); free(w_r); free(bias); free(noise); free(logits); free(idx); free(gate); free(probs); free(margin);
    free(load); free(counts); free(offsets); free(row_of); free(dropped); free(gate_eff); free(xrows);
    free(experts); free(w1); free(w2); free(w3); free(s1); free(s2); free(s3); free(hid); free(y_perm); free(y);
    free(toks); free(y2);
  }
  printf("ok\n");
  return 0;
}
