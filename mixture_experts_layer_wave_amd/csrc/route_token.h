// route_token.h: the router's per-token epilogue (softmax, selection, gates), shared by
// the router kernels and the fused small-batch route + dispatch kernel.
// (Internal header of the HIP library; not part of the C ABI.)
//
// Method ("第 5 章 model.py 精读·中：MoE 路由与专家", §5.2, §5.2.1, §5.2.2, §5.2.3; "MoE 公式到源码
// 对照" §1.1-1.2; "8.1 MoE 系列" §3 for the GShard noisy second choice).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int EP>
__device__ __forceinline__ float pick(const float (&v)[EP], int i) {
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < EP; ++e) r = (e == i) ? v[e] : r;
  return r;
}

// Epilogue of one token t < N from its logits l (bias included): noisy top-k gating,
// softmax into p, optional logits/probs outputs, the k selected experts (sel, slot 0
// first) and their gates (gt). nz: the token's E noise values (a.noise row t, or a copy
// of it), unused without noise. KM: compile-time bound on k (a.k <= KM); entries j >= KM
// of sel and gt are left untouched.
template <int EP, int KM = kMaxK>
__device__ __forceinline__ void route_token(const RouterArgs& a, int64_t t, const float* nz, float (&l)[EP],
                                            float (&p)[EP], int (&sel)[kMaxK], float (&gt)[kMaxK]) {
  const int E = a.E;
  if (a.noisy == 2) {
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (e < E) l[e] += nz[e];  // logit' = fl32(logit + noise)
  }
  float mx = l[0];
#pragma unroll
  for (int e = 1; e < EP; ++e) mx = (e < E) ? fmaxf(mx, l[e]) : mx;
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    p[e] = (e < E) ? expf(l[e] - mx) : 0.f;
    sum += p[e];
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) p[e] = p[e] / sum;

  if (a.logits_out) for (int e = 0; e < E; ++e) a.logits_out[t * E + e] = pick(l, e);
  if (a.probs_out) for (int e = 0; e < E; ++e) a.probs_out[t * E + e] = pick(p, e);

  // noisy values for slots >= 1 (GShard random routing)
  float z[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) z[e] = l[e];
  if (a.noisy == 1) {
#pragma unroll
    for (int e = 0; e < EP; ++e) z[e] = (e < E) ? l[e] + nz[e] : 0.f;
  }

  static_assert(KM >= 1 && KM <= kMaxK, "k bound");
  uint64_t chosen = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    sel[j] = 0;
    if (j < a.k) {
      const bool use_z = (j > 0) && a.noisy == 1;
      int best = -1;
      float bv = 0.f;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        const float v = use_z ? z[e] : l[e];
        const bool cand = (e < E) && !((chosen >> e) & 1ull);
        if (cand && (best < 0 || v > bv)) { best = e; bv = v; }
      }
      sel[j] = best;
      chosen |= 1ull << best;
    }
  }

  if (a.mode == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) gt[j] = (j < a.k) ? pick(p, sel[j]) : 0.f;
  } else {
    const float ref = pick(l, sel[0]);
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      gt[j] = (j < a.k) ? expf(pick(l, sel[j]) - ref) : 0.f;
      s2 += gt[j];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) gt[j] = gt[j] / s2;
  }
}

// route_token on four lanes: the quad (lanes 4i .. 4i + 3 of a wave, part = lane % 4)
// holds one token, each lane the logits l of experts EPL part .. EPL part + EPL - 1 (E <=
// 4 EPL). Same steps and selection rule as route_token; the maximum and the selection
// reduce over the quad, and the probability sum adds the lanes' partial sums as
// (s0 + s1) + (s2 + s3), so every lane of the quad ends with the same sel and gt.
// p: this lane's probabilities. nz: this lane's EPL noise values (unused without noise).
// Outputs are written only when `valid`. All four lanes must call it together.
template <int EPL, int KM = kMaxK>
__device__ __forceinline__ void route_token_quad(const RouterArgs& a, int64_t t, int part, bool valid,
                                                 const float* nz, float (&l)[EPL], float (&p)[EPL],
                                                 int (&sel)[kMaxK], float (&gt)[kMaxK]) {
  static_assert(KM >= 1 && KM <= kMaxK, "k bound");
  const int E = a.E;
  const int e0 = EPL * part;
  const int lane = lane_id();
  const int qbase = lane & ~3;
  if (a.noisy == 2) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e0 + i < E) l[i] += nz[i];  // logit' = fl32(logit + noise)
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) mx = (e0 + i < E) ? fmaxf(mx, l[i]) : mx;
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    p[i] = (e0 + i < E) ? expf(l[i] - mx) : 0.f;
    sum += p[i];
  }
  sum += __shfl_xor(sum, 1);  // lanes 0, 1: s0 + s1; lanes 2, 3: s2 + s3
  sum += __shfl_xor(sum, 2);  // (s0 + s1) + (s2 + s3) on every lane (fp32 add commutes)
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] = p[i] / sum;

  if (valid && a.logits_out)
    for (int i = 0; i < EPL && e0 + i < E; ++i) a.logits_out[t * E + e0 + i] = pick(l, i);
  if (valid && a.probs_out)
    for (int i = 0; i < EPL && e0 + i < E; ++i) a.probs_out[t * E + e0 + i] = pick(p, i);

  float z[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) z[i] = l[i];
  if (a.noisy == 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) z[i] = (e0 + i < E) ? l[i] + nz[i] : 0.f;
  }

  uint64_t chosen = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    sel[j] = 0;
    if (j < a.k) {
      const bool use_z = (j > 0) && a.noisy == 1;
      int best = -1;
      float bv = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = e0 + i;
        const float v = use_z ? z[i] : l[i];
        const bool cand = (e < E) && !((chosen >> e) & 1ull);
        if (cand && (best < 0 || v > bv)) { best = e; bv = v; }
      }
      // quad reduction: larger value wins, equal values go to the lower expert index
#pragma unroll
      for (int off = 1; off <= 2; off <<= 1) {
        const int ob = __shfl_xor(best, off);
        const float ov = __shfl_xor(bv, off);
        if (ob >= 0 && (best < 0 || ov > bv || (ov == bv && ob < best))) { best = ob; bv = ov; }
      }
      sel[j] = best;
      chosen |= 1ull << best;
    }
  }

  // value of expert e (held by quad lane e / EPL) on every lane of the quad
  auto fetch = [&](const float (&v)[EPL], int e) { return __shfl(pick(v, e % EPL), qbase + e / EPL); };
  if (a.mode == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const float g = fetch(p, sel[j]);
      gt[j] = (j < a.k) ? g : 0.f;
    }
  } else {
    const float ref = fetch(l, sel[0]);
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const float lj = fetch(l, sel[j]);
      gt[j] = (j < a.k) ? expf(lj - ref) : 0.f;
      s2 += gt[j];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) gt[j] = gt[j] / s2;
  }
}

// Stores the selection and gates of token t (a.k <= KM).
template <int KM = kMaxK>
__device__ __forceinline__ void store_topk(const RouterArgs& a, int64_t t, const int (&sel)[kMaxK],
                                           const float (&gt)[kMaxK]) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < a.k) {
      a.topk_idx[t * a.k + j] = sel[j];
      a.topk_gate[t * a.k + j] = gt[j];
    }
  }
}


}  // namespace moe
