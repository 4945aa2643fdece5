/*
 * moe_oracle.c: plain fp64 CPU oracle of the top-k Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load or call this code. It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * Every function is the plain definition of one step, written as loops over tokens and
 * experts in double precision from the exact stored input values (fp32, or bf16 bit
 * patterns widened exactly). There is no blocking, fusion or reordering; OpenMP only
 * runs independent tokens on different threads and changes no arithmetic.
 *
 * Sources (short keys used below):
 *   [GROK5]  "第 5 章 model.py 精读·中：MoE 路由与专家", https://yingwang.github.io/grok-1/05-model-2/
 *   [BOOK12] "第 12 章 MoE：路由、专家与负载", https://book.ozine.me/llm/llms-from-scratch/chapters/12_moe.html
 *   [SERIES] "8.1 MoE 系列：从 GShard 到 Mixtral，再到 Switch Transformer", https://gitcode.csdn.net/69b8cfc40a2f6a37c5980bb1.html
 *   [F2C]    "MoE 公式到源码对照", https://jerryiiii.gitbook.io/llm-review/notes/distributed/moe-formula-to-code-walkthrough
 *
 * Readings taken where the pages are silent or disagree (each is listed in the design doc):
 *   - Router decisions (selection, tie-break) are taken on fp32 logits, the precision
 *     the pages fix for the router ([GROK5] §5.2.1). Softmax and gates are then
 *     evaluated in double from those fp32 logit values.
 *   - Ties between equal fp32 values go to the lower expert index.
 *   - GShard noisy slot j>=1: argmax over unchosen experts of fl32(logit + noise)
 *     ([SERIES] §3, one noise draw per (token, expert)).
 *   - Noisy top-k gating ([GROK5] §5.2.2, logit' = logit + N(0, sigma)): every quantity
 *     after the logits (softmax, selection, gates) uses logit' = fl32(logit + noise).
 *   - Capacity slots are filled slot-major, tokens ascending within a slot; the
 *     token-major order of the [F2C] §3.2 loop is the alternative.
 *   - Switch capacity ([SERIES] §7.2): C = ceil((N / E) * CF), no k.
 *   - Drop rule for a partly dropped token: the kept slots take the whole gate mass in
 *     proportion to their gates ([SERIES] §2.2 case A, generalised).
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* Host threads used by the parallel loops (the arithmetic is the same for any count). */
int oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}

/* ---- exact widening of the stored element types ---------------------------------- */

/* A bf16 value is the upper 16 bits of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* dtype 0 = fp32, 1 = bf16 (raw 16-bit patterns). */
static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == 1) return bf16_bits_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* Expert weight W[e][r][c] of an [E][R][C] stack. dtype 0/1: the stored value. dtype 2:
 * weight-only 8-bit, the int8 value times the scale of its expert and output column,
 * s[e][c] (the dequantisation weight = weight * scales of [GROK5] §5.3.3-5.3.4; one scale per
 * expert and output column, broadcast over the input dimension). */
#define W_INT8 2
static double wel(const void* w, const float* s, int dtype, int64_t e, int64_t r, int64_t c, int64_t R, int64_t C) {
  const int64_t i = (e * R + r) * C + c;
  if (dtype == W_INT8) return (double)((const int8_t*)w)[i] * (double)s[e * C + c];
  return elem(w, dtype, i);
}

/* ---- activations ([GROK5] §5.3.5, §5.3.5.1; [BOOK12] §12.1) ------------------------ */

#define ACT_SILU 0
#define ACT_GELU_ERF 1
#define ACT_GELU_TANH 2

/* SiLU(z) = z * sigmoid(z); GELU(z) = z * Phi(z) = z/2 * (1 + erf(z / sqrt 2));
 * tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double oracle_act(int kind, double z) {
  if (kind == ACT_SILU) return z / (1.0 + exp(-z));
  if (kind == ACT_GELU_ERF) return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
  if (kind == ACT_GELU_TANH) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
  }
  return NAN;
}

/* ---- step 1: router logits ([GROK5] §5.2.1: l = x W_r in fp32) ---------------------- */

/* logits[t*E+e] = sum_d x[t,d] * w_r[d,e] + bias[e]   (bias may be NULL). */
void oracle_router_logits(int64_t N, int64_t D, int32_t E, int x_dtype, const void* x,
                          const float* w_r, const float* bias, double* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < N; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t d = 0; d < D; ++d) s += elem(x, x_dtype, t * D + d) * (double)w_r[d * E + e];
      if (bias) s += (double)bias[e];
      logits[t * E + e] = s;
    }
  }
}

/* ---- steps 2-4: softmax, top-k selection, gates -------------------------------------- */

#define MODE_SOFTMAX_TOPK 0 /* gates = full-softmax probabilities, unnormalised */
#define MODE_TOPK_SOFTMAX 1 /* gates = softmax over the selected logits          */

#define NOISE_NONE 0   /* clean top-k                                          */
#define NOISE_SECOND 1 /* GShard: slots >= 1 compare fl32(l + noise)            */
#define NOISE_ALL 2    /* noisy top-k gating: l is replaced by fl32(l + noise)  */

/* For each token t (logits are rounded to fp32 first, the router's precision; with
 * NOISE_ALL the fp32 logits are first replaced by fl32(l + noise[t,e])):
 *   probs[t,e] = exp(l_e - max l) / sum_e' exp(l_e' - max l)          ([F2C] §1.1)
 *   slot j: the unchosen expert with the largest value, lower index on ties; the value
 *   is l_e, except for slots j >= 1 under NOISE_SECOND: fl32(l_e + noise[t,e])
 *   ([GROK5] §5.2.3; [SERIES] §3)
 *   mode SOFTMAX_TOPK: gate_j = probs[t, idx_j]                        ([GROK5] §5.2.3 A)
 *   mode TOPK_SOFTMAX: gate_j = exp(l_{idx_j}) / sum_i exp(l_{idx_i})   ([BOOK12] §12.1)
 *   margin[t] = smallest, over the k selection steps, of the probability gap between the
 *   chosen expert and the best remaining one, where "probability" is the softmax over all
 *   E of the values that step compares (+inf when no expert remains). It measures how
 *   close the token is to a different selection. */
int oracle_route(int64_t N, int32_t E, int32_t k, int mode, int noisy, const double* logits,
                 const float* noise, int32_t* idx, double* gate, double* probs, double* margin) {
  if (N < 0 || E < 1 || k < 1 || k > E || E > 4096) return ORACLE_EINVAL;
  if (noisy < NOISE_NONE || noisy > NOISE_ALL || (noisy && !noise)) return ORACLE_EINVAL;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t t = 0; t < N; ++t) {
    float* l32 = (float*)malloc(sizeof(float) * E);
    float* val = (float*)malloc(sizeof(float) * E);
    double* q = (double*)malloc(sizeof(double) * E);
    unsigned char* chosen = (unsigned char*)calloc(E, 1);
    if (!l32 || !val || !q || !chosen) { bad = 1; free(l32); free(val); free(q); free(chosen); continue; }
    for (int32_t e = 0; e < E; ++e) l32[e] = (float)logits[t * E + e];
    if (noisy == NOISE_ALL)
      for (int32_t e = 0; e < E; ++e) l32[e] = l32[e] + noise[t * E + e]; /* fp32 sum, rounded once */

    /* softmax over all E experts of the fp32 logits */
    double m = l32[0];
    for (int32_t e = 1; e < E; ++e) if (l32[e] > m) m = l32[e];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) z += exp((double)l32[e] - m);
    for (int32_t e = 0; e < E; ++e) probs[t * E + e] = exp((double)l32[e] - m) / z;

    double tok_margin = INFINITY;
    for (int32_t j = 0; j < k; ++j) {
      for (int32_t e = 0; e < E; ++e)
        val[e] = (j > 0 && noisy == NOISE_SECOND) ? (float)(l32[e] + noise[t * E + e]) : l32[e];
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!chosen[e] && (best < 0 || val[e] > val[best])) best = e;
      /* probability gap to the runner-up among the remaining experts */
      double vm = val[0];
      for (int32_t e = 1; e < E; ++e) if (val[e] > vm) vm = val[e];
      double vz = 0.0;
      for (int32_t e = 0; e < E; ++e) { q[e] = exp((double)val[e] - vm); vz += q[e]; }
      int32_t second = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!chosen[e] && e != best && (second < 0 || val[e] > val[second])) second = e;
      if (second >= 0) {
        double gap = (q[best] - q[second]) / vz;
        if (gap < tok_margin) tok_margin = gap;
      }
      chosen[best] = 1;
      idx[t * k + j] = best;
    }
    if (margin) margin[t] = tok_margin;

    if (mode == MODE_SOFTMAX_TOPK) {
      for (int32_t j = 0; j < k; ++j) gate[t * k + j] = probs[t * E + idx[t * k + j]];
    } else {
      double ref = l32[idx[t * k]];
      double s = 0.0;
      for (int32_t j = 0; j < k; ++j) s += exp((double)l32[idx[t * k + j]] - ref);
      for (int32_t j = 0; j < k; ++j) gate[t * k + j] = exp((double)l32[idx[t * k + j]] - ref) / s;
    }
    free(l32); free(val); free(q); free(chosen);
  }
  return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/* ---- step 5: capacity ([F2C] §3.1; [SERIES] §2.1) ---------------------------------- */

/* formula 0: C = max(ceil(CF * N * k / E), min_capacity), the product evaluated left to
 * right in double ([F2C] §3.1).
 * formula 1: C = max(ceil((N / E) * CF), min_capacity), the Switch form without k
 * ([SERIES] §7.2: tokens per batch / experts x capacity factor).
 * Invalid inputs are an error, as in [F2C] §3.1. */
int oracle_capacity(int64_t N, int32_t E, int32_t k, double cf, int32_t min_capacity, int formula, int64_t* C) {
  if (N < 0 || E <= 0 || cf <= 0.0 || k <= 0 || min_capacity < 0 || formula < 0 || formula > 1)
    return ORACLE_EINVAL;
  double c = formula == 0 ? ceil(((cf * (double)N) * (double)k) / (double)E) : ceil(((double)N / (double)E) * cf);
  int64_t ci = (int64_t)c;
  *C = ci > min_capacity ? ci : (int64_t)min_capacity;
  return ORACLE_OK;
}

/* ---- steps 5-6: load histogram, capacity slots, drop mask ----------------------------- */

/* load[e] = #{(t,j): idx[t,j] = e}                                    ([F2C] §1.3)
 * Records are visited slot-major (tokens ascending within a slot), or token-major (slots
 * ascending within a token, the loop of [F2C] §3.2) when token_major; a record is
 * accepted while its expert holds fewer than C records, otherwise it is dropped.
 * C < 0 means no capacity limit. counts[e] = accepted records of expert e.
 * offsets[e] = e*C when padded, else the exclusive prefix sum of counts; offsets[E] = rows.
 * row_of[t,j] = offsets[e] + position, or -1 when dropped. */
int oracle_dispatch(int64_t N, int32_t E, int32_t k, const int32_t* idx, int64_t C, int padded,
                    int token_major, int64_t* load, int64_t* counts, int64_t* offsets, int64_t* row_of,
                    uint8_t* dropped) {
  if (N < 0 || E < 1 || k < 1 || (padded && C < 0)) return ORACLE_EINVAL;
  for (int32_t e = 0; e < E; ++e) { load[e] = 0; counts[e] = 0; }
  for (int64_t t = 0; t < N; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) return ORACLE_EINVAL;
      load[e] += 1;
    }
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N * k > 0 ? N * k : 1));
  if (!pos) return ORACLE_EINVAL;
  for (int64_t v = 0; v < N * k; ++v) {
    /* the v-th record in visiting order */
    const int64_t t = token_major ? v / k : v % N;
    const int32_t j = token_major ? (int32_t)(v % k) : (int32_t)(v / N);
    const int32_t e = idx[t * k + j];
    if (C < 0 || counts[e] < C) {
      pos[t * k + j] = counts[e];
      counts[e] += 1;
      dropped[t * k + j] = 0;
    } else {
      pos[t * k + j] = -1;
      dropped[t * k + j] = 1;
    }
  }
  int64_t run = 0;
  for (int32_t e = 0; e < E; ++e) {
    offsets[e] = padded ? (int64_t)e * C : run;
    run += counts[e];
  }
  offsets[E] = padded ? (int64_t)E * C : run;
  for (int64_t t = 0; t < N; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int64_t p = pos[t * k + j];
      row_of[t * k + j] = p < 0 ? -1 : offsets[idx[t * k + j]] + p;
    }
  free(pos);
  return ORACLE_OK;
}

/* ---- step 7: gates after the drop rule ([SERIES] §2.2) ------------------------------ */

/* Every slot kept: gate_eff = gate. No slot kept: gate_eff = 0 (the token passes through
 * with increment 0, case B). Otherwise the kept slots share the whole gate mass:
 * gate_eff_j = gate_j * (sum_all gate) / (sum_kept gate); dropped slots get 0 (case A,
 * which gives (1,0) for two renormalised gates). */
void oracle_drop_rule(int64_t N, int32_t k, const double* gate, const uint8_t* dropped,
                      double* gate_eff) {
  for (int64_t t = 0; t < N; ++t) {
    double all = 0.0, kept = 0.0;
    int32_t nk = 0;
    for (int32_t j = 0; j < k; ++j) {
      all += gate[t * k + j];
      if (!dropped[t * k + j]) { kept += gate[t * k + j]; nk += 1; }
    }
    for (int32_t j = 0; j < k; ++j) {
      double g = gate[t * k + j];
      if (nk == k) gate_eff[t * k + j] = g;
      else if (nk == 0 || dropped[t * k + j]) gate_eff[t * k + j] = 0.0;
      else gate_eff[t * k + j] = g * all / kept;
    }
  }
}

/* ---- step 8: one expert on one token ([BOOK12] §12.1; [GROK5] §5.3.5) ----------------- */

/* h[f] = act(sum_d x_d W1[e,d,f]) * (sum_d x_d W2[e,d,f]); W1, W2 are [E,D,F]
 * (s1, s2: [E,F] scales when w_dtype is int8, else unused). */
int oracle_expert_hidden(int64_t D, int64_t F, int w_dtype, int act, const double* x,
                         const void* w1, const float* s1, const void* w2, const float* s2, int32_t e, double* h) {
  double* h1 = (double*)calloc((size_t)F, sizeof(double));
  double* h2 = (double*)calloc((size_t)F, sizeof(double));
  if (!h1 || !h2) { free(h1); free(h2); return ORACLE_EINVAL; }
  for (int64_t d = 0; d < D; ++d) {
    const double xd = x[d];
    for (int64_t f = 0; f < F; ++f) {
      h1[f] += xd * wel(w1, s1, w_dtype, e, d, f, D, F);
      h2[f] += xd * wel(w2, s2, w_dtype, e, d, f, D, F);
    }
  }
  for (int64_t f = 0; f < F; ++f) h[f] = oracle_act(act, h1[f]) * h2[f];
  free(h1); free(h2);
  return ORACLE_OK;
}

/* out[d] = sum_f h_f W3[e,f,d] with h from oracle_expert_hidden; W3 is [E,F,D]
 * (s3: [E,D] scales when w_dtype is int8). */
int oracle_expert_ffn(int64_t D, int64_t F, int w_dtype, int act, const double* x, const void* w1,
                      const float* s1, const void* w2, const float* s2, const void* w3, const float* s3,
                      int32_t e, double* out) {
  double* h = (double*)malloc(sizeof(double) * (size_t)F);
  if (!h) return ORACLE_EINVAL;
  if (oracle_expert_hidden(D, F, w_dtype, act, x, w1, s1, w2, s2, e, h) != ORACLE_OK) { free(h); return ORACLE_EINVAL; }
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t f = 0; f < F; ++f) {
    const double u = h[f];
    for (int64_t d = 0; d < D; ++d) out[d] += u * wel(w3, s3, w_dtype, e, f, d, F, D);
  }
  free(h);
  return ORACLE_OK;
}

/* Expert outputs for a list of expert-buffer rows: out[i,:] = f_{e_i}(xrows[i,:]) and
 * hid[i,:] = the hidden vector h (either output may be NULL). */
int oracle_expert_rows(int64_t n, int64_t D, int64_t F, int w_dtype, int act, const double* xrows,
                       const int32_t* experts, const void* w1, const float* s1, const void* w2, const float* s2,
                       const void* w3, const float* s3, double* hid, double* out) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n; ++i) {
    if (hid && oracle_expert_hidden(D, F, w_dtype, act, xrows + i * D, w1, s1, w2, s2, experts[i], hid + i * F) !=
                   ORACLE_OK)
      bad = 1;
    if (out && oracle_expert_ffn(D, F, w_dtype, act, xrows + i * D, w1, s1, w2, s2, w3, s3, experts[i],
                                 out + i * D) != ORACLE_OK)
      bad = 1;
  }
  return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/* ---- step 9 (combine alone): y[t,:] = sum over slots j with row_of[t,j] >= 0, in slot
 * order, of gate_eff[t,j] * y_perm[row_of[t,j],:] ([GROK5] §5.3.5; [BOOK12] §12.2). */
void oracle_combine(int64_t N, int64_t D, int32_t k, const double* y_perm, const int64_t* row_of,
                    const double* gate_eff, double* y) {
  for (int64_t t = 0; t < N; ++t) {
    for (int64_t d = 0; d < D; ++d) y[t * D + d] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int64_t r = row_of[t * k + j];
      if (r < 0) continue;
      for (int64_t d = 0; d < D; ++d) y[t * D + d] += gate_eff[t * k + j] * y_perm[r * D + d];
    }
  }
}

/* ---- step 9: layer output for a list of tokens ([GROK5] §5.3.5, §5.8; [BOOK12] §12.2) */

/* y[i,:] = sum over kept slots j of token t = toks[i], in slot order, of
 * gate_eff[t,j] * f_{idx[t,j]}(x_t); 0 when every slot is dropped. */
int oracle_layer_tokens(int64_t n_tok, const int64_t* toks, int64_t N, int64_t D, int64_t F,
                        int32_t E, int32_t k, int dtype, int w_dtype, int act, const void* x,
                        const void* w1, const float* s1, const void* w2, const float* s2, const void* w3,
                        const float* s3, const int32_t* idx, const uint8_t* dropped, const double* gate_eff,
                        double* y) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_tok; ++i) {
    const int64_t t = toks[i];
    double* xt = (double*)malloc(sizeof(double) * (size_t)D);
    double* fo = (double*)malloc(sizeof(double) * (size_t)D);
    if (!xt || !fo || t < 0 || t >= N) { bad = 1; free(xt); free(fo); continue; }
    for (int64_t d = 0; d < D; ++d) xt[d] = elem(x, dtype, t * D + d);
    for (int64_t d = 0; d < D; ++d) y[i * D + d] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      if (dropped && dropped[t * k + j]) continue;
      const int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) { bad = 1; break; }
      if (oracle_expert_ffn(D, F, w_dtype, act, xt, w1, s1, w2, s2, w3, s3, e, fo) != ORACLE_OK) { bad = 1; break; }
      const double g = gate_eff[t * k + j];
      for (int64_t d = 0; d < D; ++d) y[i * D + d] += g * fo[d];
    }
    free(xt); free(fo);
  }
  return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/* ---- statistics ([F2C] §2.1-2.3, §3.3; [GROK5] §5.5.2) ------------------------------ */

/* P_e = (1/N) sum_t probs[t,e]; f_e = load_e / (N k);
 * balance = E * sum_e f_e P_e; balance_div_n = E * sum_e (load_e / N) P_e. */
void oracle_balance(int64_t N, int32_t E, int32_t k, const double* probs, const int64_t* load,
                    double* P, double* balance, double* balance_div_n) {
  double b = 0.0, bn = 0.0;
  for (int32_t e = 0; e < E; ++e) {
    double s = 0.0;
    for (int64_t t = 0; t < N; ++t) s += probs[t * E + e];
    P[e] = s / (double)N;
    b += ((double)load[e] / ((double)N * (double)k)) * P[e];
    bn += ((double)load[e] / (double)N) * P[e];
  }
  *balance = (double)E * b;
  *balance_div_n = (double)E * bn;
}
