// router.hip: fused router for gfx950. fp32 logits x W_r (+ bias), stable softmax over
// the E experts, register top-k, gates, and per-block partial sums of the probabilities.
//
// Method ("第 5 章 model.py 精读·中：MoE 路由与专家", §5.2, §5.2.1, §5.2.3; "MoE 公式到源码对照"
// §1.1-1.2; "8.1 MoE 系列" §3 for the GShard noisy second choice):
//   logits = fp32(x) W_r in fp32; p = softmax(logits) with the maximum subtracted;
//   slots = k largest logits (lower index wins ties), slot 0 the largest; in noisy mode
//   slots >= 1 use fl32(logit + noise) over the experts not chosen yet;
//   gates = p of the chosen experts (softmax-then-top-k) or softmax over the chosen
//   logits (top-k-then-softmax, the renormalised form).
//
// Design: a workgroup owns 64 tokens, one per lane; its 4 waves split D into quarters
// so each lane keeps E fp32 accumulators for its token. The W_r rows of the current
// chunk are staged in LDS and read as wave-wide broadcasts (every lane of a wave reads
// the same address). The four quarter sums are added in a fixed order, so logits are
// bit-reproducible. Selection runs in registers on the lane that owns the token: no
// cross-lane traffic and no atomics.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTM = kRouterTokens;  // tokens per workgroup = lanes of a wave
constexpr int kDC = 16;             // D rows per chunk per wave

template <int EP>
__device__ __forceinline__ float pick(const float (&v)[EP], int i) {
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < EP; ++e) r = (e == i) ? v[e] : r;
  return r;
}

template <typename XT>
__device__ __forceinline__ void load_chunk(const XT* p, float (&xv)[kDC]);

template <>
__device__ __forceinline__ void load_chunk<float>(const float* p, float (&xv)[kDC]) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < kDC / 4; ++i) {
    f32x4 v = q[i];
    xv[4 * i + 0] = v[0]; xv[4 * i + 1] = v[1]; xv[4 * i + 2] = v[2]; xv[4 * i + 3] = v[3];
  }
}

template <>
__device__ __forceinline__ void load_chunk<bf16>(const bf16* p, float (&xv)[kDC]) {
  const bf16x8* q = reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < kDC / 8; ++i) {
    bf16x8 v = q[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[8 * i + j] = (float)v[j];
  }
}

template <int EP, typename XT, bool FROM_LOGITS>
__global__ __launch_bounds__(256) void k_router(const RouterArgs a) {
  __shared__ float wr_s[4][kDC][EP];
  __shared__ float red_s[3][EP][kTM];
  __shared__ float ps_s[EP][kTM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int E = a.E;
  const int64_t t = (int64_t)blockIdx.x * kTM + lane;
  const bool valid = t < a.N;

  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.f;

  if constexpr (!FROM_LOGITS) {
    const int Dq = a.D / 4;
    const XT* xrow = reinterpret_cast<const XT*>(a.x) + (valid ? t : 0) * (int64_t)a.D + (int64_t)w * Dq;
    for (int c = 0; c < Dq; c += kDC) {
      for (int i = tid; i < 4 * kDC * EP; i += 256) {
        const int ww = i / (kDC * EP), r = (i / EP) % kDC, e = i % EP;
        wr_s[ww][r][e] = e < E ? a.w_r[(int64_t)(ww * Dq + c + r) * E + e] : 0.f;
      }
      __syncthreads();
      float xv[kDC];
      load_chunk<XT>(xrow + c, xv);
#pragma unroll
      for (int r = 0; r < kDC; ++r) {
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] = fmaf(xv[r], wr_s[w][r][e], acc[e]);
      }
      __syncthreads();
    }
    if (w > 0) {
#pragma unroll
      for (int e = 0; e < EP; ++e) red_s[w - 1][e][lane] = acc[e];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[e] = ((acc[e] + red_s[0][e][lane]) + red_s[1][e][lane]) + red_s[2][e][lane];
    }
  } else {
    if (w == 0 && valid) {
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[e] = e < E ? a.logits_in[t * E + e] : 0.f;
    }
  }

  if (w == 0) {
    float l[EP], p[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float b = (!FROM_LOGITS && a.bias != nullptr && e < E) ? a.bias[e] : 0.f;
      l[e] = acc[e] + b;
    }
    // stable softmax over the E experts
    float m = l[0];
#pragma unroll
    for (int e = 1; e < EP; ++e) m = (e < E) ? fmaxf(m, l[e]) : m;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      p[e] = (e < E) ? expf(l[e] - m) : 0.f;
      s += p[e];
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) p[e] = p[e] / s;

    if (valid) {
      if (a.logits_out) for (int e = 0; e < E; ++e) a.logits_out[t * E + e] = pick(l, e);
      if (a.probs_out) for (int e = 0; e < E; ++e) a.probs_out[t * E + e] = pick(p, e);

      // noisy values for slots >= 1 (GShard random routing)
      float z[EP];
#pragma unroll
      for (int e = 0; e < EP; ++e) z[e] = l[e];
      if (a.noisy) {
#pragma unroll
        for (int e = 0; e < EP; ++e) z[e] = (e < E) ? l[e] + a.noise[t * E + e] : 0.f;
      }

      int sel[kMaxK];
      uint64_t chosen = 0;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        sel[j] = 0;
        if (j < a.k) {
          const bool use_z = (j > 0) && a.noisy;
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

      float g[kMaxK];
      if (a.mode == 0) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) g[j] = (j < a.k) ? pick(p, sel[j]) : 0.f;
      } else {
        const float ref = pick(l, sel[0]);
        float s2 = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          g[j] = (j < a.k) ? expf(pick(l, sel[j]) - ref) : 0.f;
          s2 += g[j];
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) g[j] = g[j] / s2;
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < a.k) {
          a.topk_idx[t * a.k + j] = sel[j];
          a.topk_gate[t * a.k + j] = g[j];
        }
      }
    }
    if (a.psum) {
#pragma unroll
      for (int e = 0; e < EP; ++e) ps_s[e][lane] = valid ? p[e] : 0.f;
    }
  }
  if (a.psum) {
    __syncthreads();
    if (tid < E) {
      float s = 0.f;
      for (int i = 0; i < kTM; ++i) s += ps_s[tid][i];
      a.psum[(int64_t)blockIdx.x * E + tid] = s;
    }
    if (blockIdx.x == 0 && tid == 0 && a.psum_magic) *a.psum_magic = kPsumMagic;
  }
}

template <int EP>
hipError_t launch_ep(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + kTM - 1) / kTM)), block(256);
  if (a.logits_in) {
    hipLaunchKernelGGL((k_router<EP, float, true>), grid, block, 0, s, a);
  } else if (bf16_x) {
    hipLaunchKernelGGL((k_router<EP, bf16, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_router<EP, float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  if (a.E <= 8) return launch_ep<8>(a, bf16_x, s);
  if (a.E <= 16) return launch_ep<16>(a, bf16_x, s);
  if (a.E <= 32) return launch_ep<32>(a, bf16_x, s);
  return launch_ep<64>(a, bf16_x, s);
}

}  // namespace moe
