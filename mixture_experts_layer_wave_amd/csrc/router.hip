// router.hip: router of the MoE layer for gfx950. fp32 logits x W_r (+ bias), stable
// softmax over the E experts, register top-k, gates, and per-block partial sums of the
// probabilities.
//
// Method ("第 5 章 model.py 精读·中：MoE 路由与专家", §5.2, §5.2.1, §5.2.2, §5.2.3; "MoE 公式到源码
// 对照" §1.1-1.2; "8.1 MoE 系列" §3 for the GShard noisy second choice):
//   logits = fp32(x) W_r in fp32; p = softmax(logits) with the maximum subtracted;
//   slots = k largest logits (lower index wins ties), slot 0 the largest; in GShard mode
//   slots >= 1 use fl32(logit + noise) over the experts not chosen yet; in noisy top-k
//   gating logit' = fl32(logit + noise) replaces the logits for every later step;
//   gates = p of the chosen experts (softmax-then-top-k) or softmax over the chosen
//   logits (top-k-then-softmax, the renormalised form).
//
// Two logit paths, one token epilogue (route_token):
//  * Split-K path (bf16 x, scratch given): workgroups of 8 waves x 32 tokens take one
//    token tile and one of S equal ranges of D; S is chosen so that about 256 workgroups
//    run whatever N is (decode included). Products x * W_r are formed on the bf16 matrix
//    cores without losing fp32 accuracy: each fp32 W_r value is split exactly into three
//    bf16 pieces (hi + mid + lo, 8 mantissa bits each) when its 64-row chunk is staged in
//    LDS, x is bf16 already, so every product is exact and v_mfma_f32_32x32x16_bf16
//    accumulates in fp32. Partial logits [S][N][E] go to scratch; k_router_epi adds them
//    in split order (fixed, so logits are bit-reproducible) and finishes each token.
//  * Single-pass path (fp32 x, routing given logits, or no scratch): a workgroup owns 32
//    tokens, its 8 waves split D and accumulate with v_mfma_f32_32x32x2_f32; the 8
//    partial blocks meet in LDS and are added in wave order before the epilogue.
//  * Token-parallel path (bf16 x with scratch, at most kTokRouterTokens tokens, E <= 16):
//    one workgroup per token forms the whole logit row with fp32 fused multiply-adds and a
//    fixed reduction tree, then finishes the token, so a small batch needs one launch and
//    no split-K partials (the decode regime).
#include "moe_device.h"
#include "moe_internal.h"
#include "route_token.h"

namespace moe {
namespace {

constexpr int kTM = kRouterTokens;  // tokens per single-pass workgroup (32)
constexpr int kWaves = 8;
constexpr int kKC = 32;             // K chunk per pipeline step of the single-pass path

// ---- single-pass path --------------------------------------------------------------

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
template <int NT, int EP, typename XT, bool FROM_LOGITS, int KM>
__global__ __launch_bounds__(512) void k_router(const RouterArgs a) {
  __shared__ float red_s[FROM_LOGITS ? 1 : kWaves][NT][16][64];  // partial logit blocks, lane-contiguous
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
      l[e] = v;
    }
    if (valid) {
      int sel[kMaxK];
      float gt[kMaxK];
      route_token<EP, KM>(a, t, a.noise != nullptr ? a.noise + t * E : nullptr, l, p, sel, gt);
      store_topk<KM>(a, t, sel, gt);
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

// ---- split-K path (bf16 x) -----------------------------------------------------------

constexpr int kRow = kRouterChunk + 8;  // bf16 per LDS row of a W_r plane (16-byte pad)

// Exact split of an fp32 value into three bf16 pieces: v = hi + mid + lo. Each piece
// takes the next 8 significant bits; both subtractions are exact.
__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t u = __float_as_uint(v);
  const float r1 = v - __uint_as_float(u & 0xffff0000u);
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
  hi = (uint16_t)(u >> 16);
  mid = (uint16_t)(u1 >> 16);
  lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

// Workgroup (token tile, split): 8 waves x 32 tokens, K range [split Ks, (split+1) Ks).
template <int NT>
__global__ __launch_bounds__(512) void k_router_split(const RouterArgs a, RouterSplit rs) {
  constexpr int EP = 32 * NT;
  constexpr int KC = kRouterChunk;
  constexpr int PER = KC * EP / 512;  // W_r values staged per thread and chunk
  static_assert(PER * 512 == KC * EP, "staging split");
  __shared__ __attribute__((aligned(16))) uint16_t w_s[2][3][EP][kRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int E = a.E;
  const int tile = blockIdx.x / rs.S, split = blockIdx.x % rs.S;
  const int64_t t0 = (int64_t)tile * kRouterTile + 32 * w;
  const bool active = t0 < a.N;  // wave-uniform: waves past N only help staging
  const int m = lane & 31, g = lane >> 5;
  const int kbeg = split * rs.Ks;
  const int nch = rs.Ks / KC;
  // Lane (token m, group g) feeds k = 32 g + 8 s + 0..7 of MFMA step s of a chunk; the
  // W_r operand of the same lane group covers the same k.
  const int64_t trow = min(t0 + m, a.N - 1);
  const u32x4* xrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(a.x) + trow * a.D + kbeg + 32 * g);

  // Global loads run two chunks ahead: the W_r rows and x words of chunk c + 2 are
  // requested while chunk c is multiplied; chunk c + 1 goes to LDS after it.
  auto fetch_w = [&](int c, float (&wst)[PER]) {  // W_r rows of chunk c into registers
    const int k0 = kbeg + c * KC;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i;
      const int kk = q / EP, e = q % EP;
      wst[i] = e < E ? a.w_r[(int64_t)(k0 + kk) * E + e] : 0.f;
    }
  };
  auto store_w = [&](int buf, const float (&wst)[PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i;
      const int kk = q / EP, e = q % EP;
      uint16_t h, md, lo;
      split3(wst[i], h, md, lo);
      w_s[buf][0][e][kk] = h;
      w_s[buf][1][e][kk] = md;
      w_s[buf][2][e][kk] = lo;
    }
  };
  auto fetch_x = [&](int c, u32x4 (&xa)[4]) {
    if (active) {
#pragma unroll
      for (int s = 0; s < 4; ++s) xa[s] = xrow[c * (KC / 8) + s];
    }
  };

  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;

  float w0[PER], w1[PER], w2[PER];
  u32x4 x0[4], x1[4], x2[4];
  fetch_w(0, w0);
  fetch_x(0, x0);
  if (nch > 1) {
    fetch_w(1, w1);
    fetch_x(1, x1);
  }
  store_w(0, w0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 2 < nch) {
      fetch_w(c + 2, w2);
      fetch_x(c + 2, x2);
    }
    if (active) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, x0[s]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int pc = 0; pc < 3; ++pc) {
            const bf16x8 wv = *reinterpret_cast<const bf16x8*>(&w_s[buf][pc][nt * 32 + m][32 * g + 8 * s]);
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, wv, acc[nt], 0, 0, 0);
          }
      }
    }
    if (c + 1 < nch) store_w(buf ^ 1, w1);  // that buffer's last readers passed the previous barrier
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) { x0[s] = x1[s]; x1[s] = x2[s]; }
#pragma unroll
    for (int i = 0; i < PER; ++i) w1[i] = w2[i];
  }
  if (!active) return;
  // Accumulator element r of a lane holds token row 8 (r / 4) + 4 g + r % 4 and expert
  // column m of its 32 x 32 block.
  float* P = a.rpart + (int64_t)split * a.N * E;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = nt * 32 + m;
    if (e >= E) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + 8 * (r / 4) + 4 * g + (r % 4);
      if (t < a.N) P[t * E + e] = acc[nt][r];
    }
  }
}

// 64 tokens per workgroup. Phase 1: the 256 threads sum the split partials of the
// 64 x E logits, each in split order (the loads of all items of a thread and of up to
// 64 / items splits are in flight at once; consecutive threads read consecutive partials). Phase 2: one thread per token adds the
// bias and runs the token epilogue. Block sums of the probabilities per 32 tokens.
template <int EP, int KM>
__global__ __launch_bounds__(256) void k_router_epi(const RouterArgs a, RouterSplit rs) {
  __shared__ float l_s[64][EP + 1];
  __shared__ float ps_s[EP][64];
  __shared__ float nz_s[64][EP];  // the 64 tokens' noise rows (coalesced copy)
  __shared__ float b_s[EP];       // logit bias (0 without one)
  const int tid = threadIdx.x;
  const int E = a.E;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int ntok = (int)min((int64_t)64, a.N - t0);
  const int64_t stride = a.N * E;  // floats between consecutive splits
  constexpr int IT = EP / 4;                  // items (token, expert) per thread: 64 EP / 256
  constexpr int SB = IT >= 64 ? 1 : 64 / IT;  // splits whose loads are in flight together
  const int nitem = ntok * E;
  const float* P = a.rpart + t0 * E + tid;
  float v[IT];
#pragma unroll
  for (int j = 0; j < IT; ++j) v[j] = 0.f;
  for (int s0 = 0; s0 < rs.S; s0 += SB) {
    float q[SB][IT];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < IT; ++j)
        q[u][j] = (s0 + u < rs.S && tid + 256 * j < nitem) ? P[(int64_t)(s0 + u) * stride + 256 * j] : 0.f;
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < IT; ++j)
        if (s0 + u < rs.S) v[j] += q[u][j];
  }
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int i = tid + 256 * j;
    if (i < nitem) l_s[i / E][i % E] = v[j];
  }
  if (a.noise != nullptr)
    for (int i = tid; i < nitem; i += 256) nz_s[i / E][i % E] = a.noise[t0 * E + i];
  if (tid < EP) b_s[tid] = (a.bias != nullptr && tid < E) ? a.bias[tid] : 0.f;
  __syncthreads();
  {
    // four lanes per token (EP / 4 experts each): all four waves, a quarter of the chain
    constexpr int EPL = EP / 4;
    const int tok = tid >> 2, part = tid & 3;
    const int64_t t = t0 + tok;
    const bool valid = tok < ntok;
    float l[EPL], p[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = EPL * part + i;
      l[i] = (valid && e < E) ? l_s[tok][e] + b_s[e] : 0.f;
    }
    int sel[kMaxK];
    float gt[kMaxK];
    route_token_quad<EPL, KM>(a, t, part, valid, &nz_s[tok][EPL * part], l, p, sel, gt);
    if (valid && part == 0) store_topk<KM>(a, t, sel, gt);
#pragma unroll
    for (int i = 0; i < EPL; ++i) ps_s[EPL * part + i][tok] = valid ? p[i] : 0.f;
  }
  if (a.psum == nullptr) return;  // uniform
  __syncthreads();
  if (tid < E) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t blk = 2 * (int64_t)blockIdx.x + h;
      if (blk * kTM >= a.N) break;
      float s = 0.f;
      for (int i = 0; i < kTM; ++i) s += ps_s[tid][h * kTM + i];
      a.psum[blk * E + tid] = s;
    }
  }
  if (blockIdx.x == 0 && tid == 0 && a.psum_magic) *a.psum_magic = kPsumMagic;
}

// ---- token-parallel path (bf16 x, small batches) ------------------------------------

// One workgroup per token. Thread i takes rows i, i + 512, ... of D (a wave reads 64
// consecutive rows of W_r, so its loads are coalesced) and adds x[d] W_r[d][e] over them
// with fp32 fused multiply-adds in row order; the 512 partial rows are then added in a
// fixed tree (a xor butterfly over each wave's lanes, whose pairwise sums are equal on both
// lanes, then the 8 waves in order), so the logits are bit-reproducible. Lanes 0..3 of
// wave 0 finish the token with the quad epilogue and keep its probabilities in the split-K
// partial region, from which the statistics form the 32-token block sums.
template <int EP, int KM>
__global__ __launch_bounds__(512) void k_router_tok(const RouterArgs a) {
  __shared__ float red_s[kWaves][EP];
  constexpr int U = 8;  // rows per thread whose loads are in flight together (D = 4096: all)
  constexpr int EPL = EP / 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int E = a.E;
  const int64_t t = blockIdx.x;
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(a.x) + t * a.D;
  // the epilogue lanes' bias and noise values, requested before the logit loads (every
  // lane loads, at a clamped index, so no wait is needed before those loads; only lanes
  // 0..3 of wave 0 use them, for their experts below E)
  float bz[EPL], nzl[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(EPL * lane + i, E - 1);
    bz[i] = a.bias != nullptr ? a.bias[e] : 0.f;
    nzl[i] = a.noise != nullptr ? a.noise[t * E + e] : 0.f;
  }
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.f;
  for (int d0 = tid; d0 < a.D; d0 += U * 512) {
    float xf[U];
    f32x4 wq[U][EP / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // unconditional loads (rows past D re-read the last row, unused)
      const int d = min(d0 + u * 512, a.D - 1);
      xf[u] = __uint_as_float((uint32_t)xr[d] << 16);
      if (E == EP) {
#pragma unroll
        for (int q = 0; q < EP / 4; ++q) wq[u][q] = reinterpret_cast<const f32x4*>(a.w_r + (int64_t)d * E)[q];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * 512;
      if (d >= a.D) continue;
      if (E == EP) {
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] = fmaf(xf[u], wq[u][e / 4][e % 4], acc[e]);
      } else {
        const float* wrow = a.w_r + (int64_t)d * E;
#pragma unroll
        for (int e = 0; e < EP; ++e)
          if (e < E) acc[e] = fmaf(xf[u], wrow[e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EP; ++e) red_s[w][e] = acc[e];
  }
  __syncthreads();
  if (w != 0 || lane >= 4) return;
  const int part = lane;
  float l[EPL], p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = EPL * part + i;
    float v = 0.f;
    if (e < E) {
      v = red_s[0][e];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) v += red_s[ww][e];
      if (a.bias != nullptr) v += bz[i];
    }
    l[i] = v;
  }
  int sel[kMaxK];
  float gt[kMaxK];
  route_token_quad<EPL, KM>(a, t, part, true, nzl, l, p, sel, gt);
  if (part == 0) store_topk<KM>(a, t, sel, gt);
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (EPL * part + i < E) a.rpart[t * E + EPL * part + i] = p[i];
  if (t == 0 && part == 0 && a.psum_magic) *a.psum_magic = kProbsMagic;
}

// KM: compile-time bound on k for the token epilogue (2 covers the common top-1 / top-2).
template <int NT, int EP, int KM>
hipError_t launch_epk(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  if constexpr (EP <= 16) {
    if (bf16_x && a.logits_in == nullptr && a.rpart != nullptr && router_token_parallel(a.N, a.E)) {
      hipLaunchKernelGGL((k_router_tok<EP, KM>), dim3((unsigned)a.N), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  if (bf16_x && a.logits_in == nullptr && a.rpart != nullptr && a.D % kRouterChunk == 0) {
    const RouterSplit rs = router_split(a.N, a.D);
    hipLaunchKernelGGL((k_router_split<NT>), dim3((unsigned)(rs.tiles * rs.S)), dim3(512), 0, s, a, rs);
    hipLaunchKernelGGL((k_router_epi<EP, KM>), dim3((unsigned)((a.N + 63) / 64)), dim3(256), 0, s, a, rs);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.N + kTM - 1) / kTM)), block(512);
  if (a.logits_in) {
    hipLaunchKernelGGL((k_router<NT, EP, float, true, KM>), grid, block, 0, s, a);
  } else if (bf16_x) {
    hipLaunchKernelGGL((k_router<NT, EP, bf16, false, KM>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_router<NT, EP, float, false, KM>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int NT, int EP>
hipError_t launch_ep(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  return a.k <= 2 ? launch_epk<NT, EP, 2>(a, bf16_x, s) : launch_epk<NT, EP, kMaxK>(a, bf16_x, s);
}

}  // namespace

hipError_t launch_router_split(const RouterArgs& a, hipStream_t s) {
  if (a.rpart == nullptr || a.logits_in != nullptr || a.D % kRouterChunk != 0) return hipErrorInvalidValue;
  const RouterSplit rs = router_split(a.N, a.D);
  const dim3 grid((unsigned)(rs.tiles * rs.S));
  if (a.E <= 32) hipLaunchKernelGGL((k_router_split<1>), grid, dim3(512), 0, s, a, rs);
  else hipLaunchKernelGGL((k_router_split<2>), grid, dim3(512), 0, s, a, rs);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, bool bf16_x, hipStream_t s) {
  if (a.E <= 8) return launch_ep<1, 8>(a, bf16_x, s);
  if (a.E <= 16) return launch_ep<1, 16>(a, bf16_x, s);
  if (a.E <= 32) return launch_ep<1, 32>(a, bf16_x, s);
  return launch_ep<2, 64>(a, bf16_x, s);
}

}  // namespace moe
