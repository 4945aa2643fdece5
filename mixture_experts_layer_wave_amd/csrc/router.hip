// router.hip: fused router for gfx950. fp32 logits x W_r (+ bias), stable softmax over
// the E experts, register top-k, gates, and per-block partial sums of the probabilities.
//
// Method ("第 5 章 model.py 精读·中：MoE 路由与专家", §5.2, §5.2.1, §5.2.3; "MoE 公式到源码对照"
// §1.1-1.2; "8.1 MoE 系列" §3 for the GShard noisy second choice):
//   logits = fp32(x) W_r in fp32; p = softmax(logits) with the maximum subtracted;
//   slots = k largest logits (lower index wins ties), slot 0 the largest; in GShard mode
//   slots >= 1 use fl32(logit + noise) over the experts not chosen yet; in noisy top-k
//   gating ("第 5 章 ..." §5.2.2) logit' = fl32(logit + noise) replaces the logits;
//   gates = p of the chosen experts (softmax-then-top-k) or softmax over the chosen
//   logits (top-k-then-softmax, the renormalised form).
//
// Design: a workgroup owns 32 tokens and its 8 waves split D into 8 equal ranges. Each
// wave accumulates the 32 x (32 or 64) logit block of its range with v_mfma_f32_32x32x2_f32
// (fp32 products, fp32 accumulation): lane l feeds x[token l % 32][k] and
// W_r[k][expert l % 32] for the k of its half (l / 32), so W_r rows are read coalesced and
// x rows with 16-byte loads. The 8 partial blocks meet in LDS and are added in a fixed
// order (wave 0 .. 7), so logits are bit-reproducible. Softmax, selection and gates then
// run in registers on one lane per token: no cross-lane traffic and no atomics.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTM = kRouterTokens;  // tokens per workgroup (32)
constexpr int kWaves = 8;
constexpr int kKC = 32;             // K chunk per pipeline step: 16 MFMAs of K = 2

template <int EP>
__device__ __forceinline__ float pick(const float (&v)[EP], int i) {
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < EP; ++e) r = (e == i) ? v[e] : r;
  return r;
}

// Raw chunk of kKC x elements (as 16-byte words) and the W_r values one lane needs.
template <typename XT>
struct XChunk {
  static constexpr int kWords = kKC * sizeof(XT) / 16;
  u32x4 w[kWords];
  __device__ __forceinline__ void load(const XT* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = q[i];
  }
  __device__ __forceinline__ float at(int i) const {  // element i as fp32 (i constant)
    if constexpr (sizeof(XT) == 2) {
      const uint32_t u = w[i / 8][(i % 8) / 2];
      return __uint_as_float((i & 1) ? (u & 0xffff0000u) : (u << 16));
    } else {
      return __uint_as_float(w[i / 4][i % 4]);
    }
  }
};

// NT: 32-expert column tiles (E <= 32 * NT); EP: register array width of the epilogue.
template <int NT, int EP, typename XT, bool FROM_LOGITS>
__global__ __launch_bounds__(512) void k_router(const RouterArgs a) {
  __shared__ float red_s[kWaves][NT][16][64];  // partial logit blocks, lane-contiguous
  __shared__ float ps_s[EP][kTM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int E = a.E;
  const int64_t t0 = (int64_t)blockIdx.x * kTM;

  if constexpr (!FROM_LOGITS) {
    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
    const int m = lane & 31, g = lane >> 5;
    const int64_t trow = min(t0 + m, a.N - 1);  // tail tokens re-read a valid row
    const int Dw = a.D / kWaves;                 // a multiple of 16
    const XT* xrow = reinterpret_cast<const XT*>(a.x) + trow * (int64_t)a.D + (int64_t)w * Dw;
    const float* wr = a.w_r + (int64_t)w * Dw * E;
    // Two chunks in flight: the loads of chunk c + kKC are issued before the MFMAs of c.
    XChunk<XT> xc[2];
    float wv[2][kKC / 2][NT];
    auto load = [&](int buf, int c) {
      xc[buf].load(xrow + c);
#pragma unroll
      for (int s = 0; s < kKC / 2; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int e = nt * 32 + m;
          wv[buf][s][nt] = e < E ? wr[(int64_t)(c + 2 * s + g) * E + e] : 0.f;
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int s = 0; s < kKC / 2; ++s) {
        const float xa = g ? xc[buf].at(2 * s + 1) : xc[buf].at(2 * s);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, wv[buf][s][nt], acc[nt], 0, 0, 0);
      }
    };
    // Dw is a multiple of 16; a final partial chunk is handled 16 at a time below.
    const int full = Dw / kKC * kKC;
    if (full > 0) load(0, 0);
    for (int c = 0; c < full; c += 2 * kKC) {
      if (c + kKC < full) load(1, c + kKC);
      compute(0);
      if (c + kKC < full) {
        if (c + 2 * kKC < full) load(0, c + 2 * kKC);
        compute(1);
      }
    }
    for (int c = full; c < Dw; c += 16) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int k = c + 2 * s + g;
        const float xa = (float)xrow[k];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int e = nt * 32 + m;
          const float wb = e < E ? wr[(int64_t)k * E + e] : 0.f;
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, wb, acc[nt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) red_s[w][nt][r][lane] = acc[nt][r];
  }
  __syncthreads();

  // Epilogue: lane t (< 32) of wave 0 owns token t0 + t.
  float p[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) p[e] = 0.f;
  const int64_t t = t0 + lane;
  const bool valid = (w == 0) && (lane < kTM) && (t < a.N);
  if (w == 0 && lane < kTM) {
    float l[EP];
    // Accumulator element r of lane l' holds row 8 (r / 4) + 4 (l' / 32) + r % 4 and
    // column l' % 32 of the 32 x 32 block.
    const int r_of = 4 * (lane >> 3) + (lane & 3);
    const int lhi = 32 * ((lane >> 2) & 1);
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float v = 0.f;
      if (e < E) {
        if constexpr (FROM_LOGITS) {
          v = valid ? a.logits_in[t * E + e] : 0.f;
        } else {
          const int nt = e / 32, n = e % 32;
          v = red_s[0][nt][r_of][lhi + n];
#pragma unroll
          for (int ww = 1; ww < kWaves; ++ww) v += red_s[ww][nt][r_of][lhi + n];
          if (a.bias != nullptr) v += a.bias[e];
        }
      }
      if (a.noisy == 2 && e < E && t < a.N) v += a.noise[t * E + e];  // noisy top-k gating: logit'
      l[e] = v;
    }
    // stable softmax over the E experts
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

    if (valid) {
      if (a.logits_out) for (int e = 0; e < E; ++e) a.logits_out[t * E + e] = pick(l, e);
      if (a.probs_out) for (int e = 0; e < E; ++e) a.probs_out[t * E + e] = pick(p, e);

      // noisy values for slots >= 1 (GShard random routing)
      float z[EP];
#pragma unroll
      for (int e = 0; e < EP; ++e) z[e] = l[e];
      if (a.noisy == 1) {
#pragma unroll
        for (int e = 0; e < EP; ++e) z[e] = (e < E) ? l[e] + a.noise[t * E + e] : 0.f;
      }

      int sel[kMaxK];
      uint64_t chosen = 0;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
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

      float gt[kMaxK];
      if (a.mode == 0) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) gt[j] = (j < a.k) ? pick(p, sel[j]) : 0.f;
      } else {
        const float ref = pick(l, sel[0]);
        float s2 = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          gt[j] = (j < a.k) ? expf(pick(l, sel[j]) - ref) : 0.f;
          s2 += gt[j];
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) gt[j] = gt[j] / s2;
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < a.k) {
          a.topk_idx[t * a.k + j] = sel[j];
          a.topk_gate[t * a.k + j] = gt[j];
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

template <int NT, int EP>
hipError_t launch_ep(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + kTM - 1) / kTM)), block(512);
  if (a.logits_in) {
    hipLaunchKernelGGL((k_router<NT, EP, float, true>), grid, block, 0, s, a);
  } else if (bf16_x) {
    hipLaunchKernelGGL((k_router<NT, EP, bf16, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_router<NT, EP, float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  if (a.E <= 8) return launch_ep<1, 8>(a, bf16_x, s);
  if (a.E <= 16) return launch_ep<1, 16>(a, bf16_x, s);
  if (a.E <= 32) return launch_ep<1, 32>(a, bf16_x, s);
  return launch_ep<2, 64>(a, bf16_x, s);
}

}  // namespace moe
