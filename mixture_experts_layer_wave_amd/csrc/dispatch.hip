// dispatch.hip: expert load histogram, slot-major capacity positions, drop rule,
// gather into expert-contiguous buffers, and the statistics reduction, for gfx950.
//
// Method ("MoE 公式到源码对照" §1.3 load histogram, §3.1-3.3 capacity, dropped mask and drop
// rate; "8.1 MoE 系列" §2.1-2.3 capacity, overflow cases A/B and zero-padded buffers;
// "第 12 章 MoE：路由、专家与负载" §12.2 expert-grouped buffers, N*k records):
//   load[e] counts the (token, slot) records of expert e. Positions inside an expert are
//   assigned slot-major (all slot-0 records in token order, then slot 1, ...) or, on
//   request, token-major (the dispatch_to_experts loop of "MoE 公式到源码对照" §3.2:
//   token by token, slots ascending); a record is kept iff its position is below C. A token whose kept slots are a
//   strict subset keeps the whole gate mass on them; a token with none kept contributes 0.
//
// Design: deterministic by construction, with no global atomics. Three passes over
// "segments" (one per slot in slot-major order; a single segment of all slots in
// token-major order):
//   count  : each 256-token workgroup builds, per segment, its expert histogram with one
//            wave ballot per expert (rank = popcount of lower lanes with equal expert);
//   scan   : one workgroup of 16 waves; each wave scans the block histograms of its
//            experts in (segment, block) order (stored expert-major, so 64 consecutive
//            entries per load and a wave prefix sum per 64), giving each block's base
//            position, the loads and counts; then one wave scans the counts into offsets;
//   assign : the same ballots give each record's rank inside its block; position =
//            base + rank. Rows, drop mask and gates after the drop rule are written.
// The gather then copies token rows into the expert buffers with 16-byte vector moves.
// Small batches (at most one 256-token block, e.g. decode) take one fused kernel instead:
// every workgroup rebuilds the whole routing table in LDS (the same ballots and scan, a few
// hundred records), workgroup 0 writes the metadata, and each workgroup gathers its share
// of the rows, so the stage is one launch with the same results.
#include "moe_device.h"
#include "moe_internal.h"
#include "route_token.h"

namespace moe {
namespace {

constexpr int kTB = kDispatchTokens;

// Per-wave match of expert ids: on return rank = number of lower lanes of this wave with
// the same expert, and cnt_s[w][x] = lanes of wave w holding expert x (x < E).
__device__ __forceinline__ void wave_match(int e, int E, int (*cnt_s)[kMaxE], int& rank) {
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  const uint64_t lt = lanemask_lt();
  rank = 0;
  for (int x = 0; x < E; ++x) {
    const uint64_t m = __ballot(e == x);
    if (e == x) rank = __popcll(m & lt);
    if (lane == 0) cnt_s[w][x] = __popcll(m);
  }
}

// Token-major match over all k slots of each lane's token: on return rank[j] = records of
// expert e[j] in lower lanes (any slot) plus those in earlier slots of the same lane, and
// cnt_s[w][x] = records of expert x in wave w.
template <int KM = kMaxK>
__device__ __forceinline__ void wave_match_tokens(const int (&e)[kMaxK], int k, int E, int (*cnt_s)[kMaxE],
                                                  int (&rank)[kMaxK]) {
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < KM; ++j) rank[j] = 0;
  for (int x = 0; x < E; ++x) {
    int c = 0, below = 0;
    for (int j = 0; j < k; ++j) {
      const uint64_t m = __ballot(e[j] == x);
      c += __popcll(m);
      below += __popcll(m & lt);
    }
    int same = 0;  // earlier slots of this lane with expert x
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k && e[j] == x) {
        rank[j] = below + same;
        ++same;
      }
    }
    if (lane == 0) cnt_s[w][x] = c;
  }
}

template <int KM = kMaxK>
__device__ __forceinline__ void load_experts(const DispatchArgs& a, int64_t t, bool valid, int (&e)[kMaxK]) {
#pragma unroll
  for (int j = KM; j < kMaxK; ++j) e[j] = -1;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    int v = (valid && j < a.k) ? a.topk_idx[t * a.k + j] : -1;
    if (v >= a.E) v = -1;  // out-of-range ids are ignored (they never index LDS or scratch)
    e[j] = v;
  }
}

__global__ __launch_bounds__(256) void k_dispatch_count(const DispatchArgs a) {
  __shared__ int cnt_s[4][kMaxE];
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kTB + tid;
  const bool valid = t < a.N;
  if (a.token_major) {
    int e[kMaxK], rank[kMaxK];
    load_experts(a, t, valid, e);
    wave_match_tokens(e, a.k, a.E, cnt_s, rank);
    __syncthreads();
    if (tid < a.E)
      a.blockcnt[(int64_t)tid * a.nblk + blockIdx.x] = cnt_s[0][tid] + cnt_s[1][tid] + cnt_s[2][tid] + cnt_s[3][tid];
    return;
  }
  for (int j = 0; j < a.k; ++j) {
    int e = valid ? a.topk_idx[t * a.k + j] : -1;
    if (e >= a.E) e = -1;  // out-of-range ids are ignored (they never index LDS or scratch)
    int rank;
    wave_match(e, a.E, cnt_s, rank);
    __syncthreads();
    if (tid < a.E)
      a.blockcnt[((int64_t)tid * a.k + j) * a.nblk + blockIdx.x] =
          cnt_s[0][tid] + cnt_s[1][tid] + cnt_s[2][tid] + cnt_s[3][tid];
    __syncthreads();
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

constexpr int kScanWaves = 16;

__global__ __launch_bounds__(64 * kScanWaves) void k_dispatch_scan(const DispatchArgs a) {
  __shared__ int cnt_s[kMaxE];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nseg = a.token_major ? 1 : a.k;
  const int64_t len = (int64_t)nseg * a.nblk;  // (segment, block) entries per expert
  // Short sequences (<= 512 entries): lane l holds entries 8 l .. 8 l + 7 of each of this
  // wave's experts (all loads issued together); a running sum inside the lane and one
  // wave scan of the lane totals per expert give the exclusive prefixes.
  constexpr int kPer = kMaxE / kScanWaves;
  if (len <= 8 * 64) {
    int v[kPer][8];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = w + kScanWaves * i;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = 8 * lane + u;
        v[i][u] = (e < a.E && q < len) ? a.blockcnt[(int64_t)e * len + q] : 0;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = w + kScanWaves * i;
      if (e >= a.E) break;
      int tot = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) tot += v[i][u];
      const int incl = wave_incl_scan(tot);
      int run_l = incl - tot;  // entries of lower lanes
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = 8 * lane + u;
        if (q < len) a.base[(int64_t)e * len + q] = run_l;
        run_l += v[i][u];
      }
      const int run = __shfl(incl, 63);
      if (lane == 0) {
        a.load[e] = run;
        a.load_copy[e] = run;
        const int c = (a.C < 0 || run < a.C) ? run : (int)a.C;
        a.counts[e] = c;
        cnt_s[e] = c;
      }
    }
  } else
  for (int e = w; e < a.E; e += kScanWaves) {
    const int32_t* cnt = a.blockcnt + (int64_t)e * len;
    int32_t* base = a.base + (int64_t)e * len;
    int run = 0;
    for (int64_t c0 = 0; c0 < len; c0 += 8 * 64) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = c0 + 64 * u + lane;
        v[u] = q < len ? cnt[q] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int incl = wave_incl_scan(v[u]);
        const int64_t q = c0 + 64 * u + lane;
        if (q < len) base[q] = run + incl - v[u];
        run += __shfl(incl, 63);
      }
    }
    if (lane == 0) {
      a.load[e] = run;
      a.load_copy[e] = run;
      const int c = (a.C < 0 || run < a.C) ? run : (int)a.C;
      a.counts[e] = c;
      cnt_s[e] = c;
    }
  }
  __syncthreads();
  if (w == 0) {
    const int c = lane < a.E ? cnt_s[lane] : 0;
    const int incl = wave_incl_scan(c);
    if (lane < a.E) a.offsets[lane] = a.padded ? (int)((int64_t)lane * a.C) : incl - c;
    if (lane == 63) a.offsets[a.E] = a.padded ? (int)((int64_t)a.E * a.C) : incl;
  }
}

__global__ __launch_bounds__(256) void k_dispatch_assign(const DispatchArgs a) {
  __shared__ int cnt_s[4][kMaxE];
  __shared__ int drop_s[4];
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int64_t t = (int64_t)blockIdx.x * kTB + tid;
  const bool valid = t < a.N;

  int row[kMaxK];
  bool kept[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) { row[j] = -1; kept[j] = false; }

  // position = base of (segment, block, expert) + records of the expert in lower waves
  // of the block + rank inside the wave; kept iff below C.
  auto place = [&](int j, int e, int seg, int rank) {
    int prefix = 0;
    for (int ww = 0; ww < w; ++ww) prefix += cnt_s[ww][e];
    const int64_t pos = (int64_t)a.base[((int64_t)e * (a.token_major ? 1 : a.k) + seg) * a.nblk + blockIdx.x] + prefix + rank;
    const bool k_ok = (a.C < 0) || (pos < a.C);
    int r = -1;
    if (k_ok) {
      const int off = a.padded ? (int)((int64_t)e * a.C) : a.offsets[e];
      r = off + (int)pos;
    }
#pragma unroll
    for (int jj = 0; jj < kMaxK; ++jj)
      if (jj == j) { row[jj] = r; kept[jj] = k_ok; }
  };

  if (a.token_major) {
    int e[kMaxK], rank[kMaxK];
    load_experts(a, t, valid, e);
    wave_match_tokens(e, a.k, a.E, cnt_s, rank);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < a.k && e[j] >= 0) place(j, e[j], 0, rank[j]);
    __syncthreads();
  } else
  for (int j = 0; j < a.k; ++j) {
    int e = valid ? a.topk_idx[t * a.k + j] : -1;
    if (e >= a.E) e = -1;  // out-of-range ids are treated as dropped records
    int rank;
    wave_match(e, a.E, cnt_s, rank);
    __syncthreads();
    if (e >= 0) place(j, e, j, rank);
    __syncthreads();
  }

  bool all_dropped = false;
  if (valid) {
    float g[kMaxK];
    float all = 0.f, ksum = 0.f;
    int nk = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      g[j] = (j < a.k) ? a.topk_gate[t * a.k + j] : 0.f;
      if (j < a.k) {
        all += g[j];
        if (kept[j]) { ksum += g[j]; nk += 1; }
      }
    }
    all_dropped = (nk == 0);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < a.k) {
        float ge;
        if (nk == a.k) ge = g[j];
        else if (nk == 0 || !kept[j]) ge = 0.f;
        else ge = g[j] * all / ksum;
        a.row_of[t * a.k + j] = row[j];
        a.dropped[t * a.k + j] = kept[j] ? 0 : 1;
        a.gate_eff[t * a.k + j] = ge;
        if (kept[j]) a.token_of_row[row[j]] = (int32_t)t;
      }
    }
  }
  const uint64_t m = __ballot(all_dropped);
  if ((tid & 63) == 0) drop_s[w] = __popcll(m);
  __syncthreads();
  if (tid == 0) a.tokdrop[blockIdx.x] = drop_s[0] + drop_s[1] + drop_s[2] + drop_s[3];
}

// Copy of one expert-buffer row by one wave: token t's row of x, or zeros (t < 0).
template <int VB>
__device__ __forceinline__ void gather_row(const GatherArgs& a, int64_t r, int64_t t, int lane) {
  const int64_t row_bytes = (int64_t)a.D * a.elem_bytes;
  const int nvec = (int)(row_bytes / VB);
  u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.x_perm) + r * row_bytes);
  if (t >= 0 && t < a.N) {
    // up to kU vectors per lane in flight before the first store, so a row costs about one
    // memory latency instead of one per vector
    constexpr int kU = 8;
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.x) + t * row_bytes);
    for (int i0 = lane; i0 < nvec; i0 += 64 * kU) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + 64 * u < nvec) v[u] = src[i0 + 64 * u];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + 64 * u < nvec) dst[i0 + 64 * u] = v[u];
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = lane; i < nvec; i += 64) dst[i] = z;
  }
}

// Fused dispatch of at most kDispatchTokens tokens (one token per thread) and at most
// kSmallRows buffer rows. Every workgroup computes the same positions: per segment (slot,
// or all slots when token-major) the ballot ranks inside each wave, then for each expert a
// running sum over (segment, wave) gives the first position of each wave's records, as the
// three-pass path does over (segment, block).
// e[j] / gt[j]: the experts (-1: none) and gates of this thread's token t = threadIdx.x.
template <int KM>
__device__ __forceinline__ void dispatch_small_body(const DispatchArgs& a, const GatherArgs& g, int (&e)[kMaxK],
                                                    const float (&gt)[kMaxK]) {
  __shared__ int cnt_s[KM][4][kMaxE];
  __shared__ int base_s[KM][4][kMaxE];
  __shared__ int cap_s[kMaxE];
  __shared__ int off_s[kMaxE + 1];
  __shared__ int tor_s[kSmallRows];
  __shared__ int drop_s[4];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int t = tid;
  const bool valid = t < a.N;
  const bool writer = blockIdx.x == 0;
  const int nseg = a.token_major ? 1 : a.k;

  int rank[kMaxK];
  if (a.token_major) {
    wave_match_tokens<KM>(e, a.k, a.E, cnt_s[0], rank);
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < a.k) wave_match(e[j], a.E, cnt_s[j], rank[j]);
  }
  for (int r = tid; r < g.rows; r += 256) tor_s[r] = -1;
  __syncthreads();
  if (tid < a.E) {
    int run = 0;
    for (int sg = 0; sg < nseg; ++sg)
      for (int ww = 0; ww < 4; ++ww) {
        base_s[sg][ww][tid] = run;
        run += cnt_s[sg][ww][tid];
      }
    const int c = (a.C < 0 || run < a.C) ? run : (int)a.C;
    cap_s[tid] = c;
    if (writer) {
      a.load[tid] = run;
      a.load_copy[tid] = run;
      a.counts[tid] = c;
    }
  }
  __syncthreads();
  if (w == 0) {
    const int c = lane < a.E ? cap_s[lane] : 0;
    const int incl = wave_incl_scan(c);
    if (lane < a.E) off_s[lane] = a.padded ? (int)((int64_t)lane * a.C) : incl - c;
    if (lane == 63) off_s[a.E] = a.padded ? (int)((int64_t)a.E * a.C) : incl;
  }
  __syncthreads();
  if (writer && tid <= a.E) a.offsets[tid] = off_s[tid];

  int row[kMaxK];
  bool kept[kMaxK];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    row[j] = -1;
    kept[j] = false;
    if (j < a.k && e[j] >= 0) {
      const int pos = base_s[a.token_major ? 0 : j][w][e[j]] + rank[j];
      kept[j] = (a.C < 0) || (pos < a.C);
      if (kept[j]) {
        row[j] = off_s[e[j]] + pos;
        tor_s[row[j]] = t;
      }
    }
  }

  bool all_dropped = false;
  if (valid) {
    float all = 0.f, ksum = 0.f;
    int nk = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < a.k) {
        all += gt[j];
        if (kept[j]) { ksum += gt[j]; nk += 1; }
      }
    }
    all_dropped = (nk == 0);
    if (writer) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < a.k) {
          float ge;
          if (nk == a.k) ge = gt[j];
          else if (nk == 0 || !kept[j]) ge = 0.f;
          else ge = gt[j] * all / ksum;
          a.row_of[t * a.k + j] = row[j];
          a.dropped[t * a.k + j] = kept[j] ? 0 : 1;
          a.gate_eff[t * a.k + j] = ge;
        }
      }
    }
  }
  const uint64_t m = __ballot(all_dropped);
  if (lane == 0) drop_s[w] = __popcll(m);
  __syncthreads();
  if (writer) {
    if (tid == 0) a.tokdrop[0] = drop_s[0] + drop_s[1] + drop_s[2] + drop_s[3];
    for (int r = tid; r < g.rows; r += 256) a.token_of_row[r] = tor_s[r];
  }
  for (int64_t r = (int64_t)blockIdx.x * 4 + w; r < g.rows; r += (int64_t)gridDim.x * 4)
    gather_row<16>(g, r, tor_s[r], lane);
}

template <int KM>
__global__ __launch_bounds__(256) void k_dispatch_small(const DispatchArgs a, const GatherArgs g) {
  const int64_t t = threadIdx.x;
  const bool valid = t < a.N;
  int e[kMaxK];
  float gt[kMaxK];
  load_experts<KM>(a, t, valid, e);
#pragma unroll
  for (int j = 0; j < KM; ++j) gt[j] = (valid && j < a.k) ? a.topk_gate[t * a.k + j] : 0.f;
  dispatch_small_body<KM>(a, g, e, gt);
}

// Route epilogue and dispatch of at most kDispatchTokens tokens in one launch (the layer's
// forward with bf16 x): every workgroup adds the S split-K partial logits of every token
// in split order and runs the token epilogue, as k_router_epi does, then dispatches as
// k_dispatch_small. Workgroup 0 also stores the selection, the gates and the probability
// block sums, so the results equal those of the separate router and dispatch calls.
template <int EP, int KM>
__global__ __launch_bounds__(256) void k_route_dispatch_small(const RouterArgs ra, int S, const DispatchArgs a,
                                                              const GatherArgs g) {
  __shared__ float l_s[kDispatchTokens][EP + 1];
  __shared__ float ps_s[EP][kDispatchTokens];
  __shared__ float nz_s[kDispatchTokens][EP];  // the tokens' noise rows (coalesced copy)
  __shared__ float b_s[EP];                    // logit bias (0 without one)
  const int tid = threadIdx.x;
  const int E = ra.E;
  const int64_t items = ra.N * E;
  const int64_t stride = ra.N * E;  // floats between consecutive splits
  // Split partials of every token, summed in split order: four consecutive items per
  // thread with one 16-byte load per split when the layout allows it, else two items per
  // thread; 32 splits' loads in flight together.
  constexpr int SB = 32, IPB = 2;
  if ((items & 3) == 0 && (stride & 3) == 0) {
    // four consecutive items per thread, one 16-byte load per split
    for (int64_t i4 = 4 * (int64_t)tid; i4 < items; i4 += 4 * 256) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < S; s0 += SB) {
        f32x4 q[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u)
          q[u] = s0 + u < S ? *reinterpret_cast<const f32x4*>(ra.rpart + (int64_t)(s0 + u) * stride + i4)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < SB; ++u)
          if (s0 + u < S) v += q[u];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) l_s[(i4 + c) / E][(i4 + c) % E] = v[c];
    }
  } else {
    for (int64_t it0 = tid; it0 < items; it0 += 256 * IPB) {
      float v[IPB];
#pragma unroll
      for (int b = 0; b < IPB; ++b) v[b] = 0.f;
      for (int s0 = 0; s0 < S; s0 += SB) {
        float q[IPB][SB];
#pragma unroll
        for (int b = 0; b < IPB; ++b)
#pragma unroll
          for (int u = 0; u < SB; ++u)
            q[b][u] = (s0 + u < S && it0 + 256 * b < items) ? ra.rpart[(int64_t)(s0 + u) * stride + it0 + 256 * b] : 0.f;
#pragma unroll
        for (int b = 0; b < IPB; ++b)
#pragma unroll
          for (int u = 0; u < SB; ++u)
            if (s0 + u < S) v[b] += q[b][u];
      }
#pragma unroll
      for (int b = 0; b < IPB; ++b) {
        const int64_t it = it0 + 256 * b;
        if (it < items) l_s[it / E][it % E] = v[b];
      }
    }
  }
  if (ra.noise != nullptr)
    for (int64_t i = tid; i < items; i += 256) nz_s[i / E][i % E] = ra.noise[i];
  if (tid < EP) b_s[tid] = (ra.bias != nullptr && tid < E) ? ra.bias[tid] : 0.f;
  __syncthreads();
  // Token epilogue on four lanes per token (EP / 4 experts each), 64 tokens per pass, as
  // k_router_epi does; each token's selection and gates go through LDS to its dispatch
  // thread (thread t holds token t below).
  __shared__ int e_s[kDispatchTokens][KM];
  __shared__ float g_s[kDispatchTokens][KM];
  constexpr int EPL = EP / 4;
  for (int64_t t0 = 0; t0 < ra.N; t0 += 64) {
    const int tok = (int)t0 + (tid >> 2), part = tid & 3;
    const bool tv = tok < ra.N;
    float l[EPL], p[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int x = EPL * part + i;
      l[i] = (tv && x < E) ? l_s[tok][x] + b_s[x] : 0.f;
    }
    int sel[kMaxK];
    float gq[kMaxK];
    route_token_quad<EPL, KM>(ra, tok, part, tv, &nz_s[tok][EPL * part], l, p, sel, gq);
    if (tv && part == 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        e_s[tok][j] = sel[j];
        g_s[tok][j] = gq[j];
      }
      if (blockIdx.x == 0) store_topk<KM>(ra, tok, sel, gq);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (tok < kDispatchTokens) ps_s[EPL * part + i][tok] = tv ? p[i] : 0.f;
  }
  __syncthreads();
  const int64_t t = tid;
  const bool valid = t < ra.N;
  int e[kMaxK];
  float gt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    e[j] = (valid && j < KM && j < a.k) ? e_s[t][j < KM ? j : 0] : -1;
    gt[j] = (valid && j < KM && j < a.k) ? g_s[t][j < KM ? j : 0] : 0.f;
  }
  if (ra.psum != nullptr) {
    __syncthreads();
    // block sums of the probabilities per kRouterTokens tokens, in token order
    if (blockIdx.x == 0 && tid < E) {
      for (int64_t blk = 0; blk * kRouterTokens < ra.N; ++blk) {
        float sum = 0.f;
        for (int i = 0; i < kRouterTokens; ++i) sum += ps_s[tid][blk * kRouterTokens + i];
        ra.psum[blk * E + tid] = sum;
      }
    }
    if (blockIdx.x == 0 && tid == 0 && ra.psum_magic) *ra.psum_magic = kPsumMagic;
  }
  dispatch_small_body<KM>(a, g, e, gt);
}

// One wave per expert-buffer row: copy the token's row or write zeros for padding.
template <int VB>  // bytes per vector move
__global__ __launch_bounds__(256) void k_gather(const GatherArgs a) {
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + w;
  if (r >= a.rows) return;
  bool valid = true;
  if (a.padded) {
    const int64_t e = r / a.C;
    valid = (r - e * a.C) < a.counts[e];
  }
  const int64_t t = valid ? (int64_t)a.token_of_row[r] : -1;
  gather_row<VB>(a, r, t, lane);
  if (!(t >= 0 && t < a.N) && lane == 0) a.token_of_row[r] = -1;
}

// Statistics of the last route + dispatch, reduced in a fixed order (double precision).
struct DevStats {
  int64_t routed_slots, dropped_slots, dropped_tokens, capacity;
  double drop_rate, token_drop_rate, balance_loss, balance_loss_div_n;
};

__global__ __launch_bounds__(64) void k_stats(const StatsArgs a) {
  __shared__ double P_s[kMaxE];
  const int e = threadIdx.x;
  const uint32_t magic = *a.psum_magic;
  const bool have_probs = magic == kProbsMagic && a.probs != nullptr;
  const bool have_p = magic == kPsumMagic || have_probs;
  if (e < a.E) {
    // sum of the block sums in block order; 16 loads in flight ahead of the adds
    double s = 0.0;
    if (have_probs) {
      // token-parallel router: the 32-token block sums formed here, in token order
      for (int64_t b = 0; b < a.nblk_r; ++b) {
        float bs = 0.f;
        for (int i = 0; i < kRouterTokens; ++i) {
          const int64_t t = b * kRouterTokens + i;
          if (t < a.N) bs += a.probs[t * a.E + e];
        }
        s += (double)bs;
      }
    } else if (have_p) {
      constexpr int U = 16;
      for (int b0 = 0; b0 < a.nblk_r; b0 += U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = a.psum[(int64_t)min(b0 + u, a.nblk_r - 1) * a.E + e];  // unconditional
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (b0 + u < a.nblk_r) s += (double)v[u];
      }
    }
    P_s[e] = s / (double)a.N;
  }
  // tokens with every slot dropped: integer sum over the dispatch blocks, spread over the wave
  int64_t dtok_l = 0;
  for (int b = e; b < a.nblk_d; b += 64) dtok_l += a.tokdrop[b];
  for (int off = 32; off > 0; off >>= 1) dtok_l += __shfl_down(dtok_l, off);
  __syncthreads();
  if (e == 0) {
    DevStats st;
    int64_t dslots = 0;
    double bal = 0.0, baln = 0.0;
    for (int x = 0; x < a.E; ++x) {
      const int64_t l = a.load[x];
      if (a.C >= 0 && l > a.C) dslots += l - a.C;
      bal += ((double)l / ((double)a.N * (double)a.k)) * P_s[x];
      baln += ((double)l / (double)a.N) * P_s[x];
    }
    const int64_t dtok = dtok_l;
    st.routed_slots = a.N * a.k;
    st.dropped_slots = dslots;
    st.dropped_tokens = dtok;
    st.capacity = a.C < 0 ? a.N : a.C;
    st.drop_rate = (double)dslots / ((double)a.N * (double)a.k);
    st.token_drop_rate = (double)dtok / (double)a.N;
    st.balance_loss = have_p ? (double)a.E * bal : 0.0;
    st.balance_loss_div_n = have_p ? (double)a.E * baln : 0.0;
    *reinterpret_cast<DevStats*>(a.out) = st;
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_dispatch_count, dim3(a.nblk), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(64 * kScanWaves), 0, s, a);
  hipLaunchKernelGGL(k_dispatch_assign, dim3(a.nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dispatch_small(const DispatchArgs& a, const GatherArgs& g, hipStream_t s) {
  if (a.N > kDispatchTokens || g.rows > kSmallRows) return hipErrorInvalidValue;
  int64_t grid = (g.rows + 3) / 4;
  grid = grid < 1 ? 1 : (grid > 256 ? 256 : grid);
  if (a.k <= 2) hipLaunchKernelGGL(k_dispatch_small<2>, dim3((unsigned)grid), dim3(256), 0, s, a, g);
  else hipLaunchKernelGGL(k_dispatch_small<kMaxK>, dim3((unsigned)grid), dim3(256), 0, s, a, g);
  return hipGetLastError();
}

hipError_t launch_route_dispatch_small(const RouterArgs& ra, const DispatchArgs& a, const GatherArgs& g,
                                       hipStream_t s) {
  if (a.N > kDispatchTokens || g.rows > kSmallRows || ra.E > 16 || ra.rpart == nullptr || ra.logits_out != nullptr ||
      ra.probs_out != nullptr)
    return hipErrorInvalidValue;
  const RouterSplit rs = router_split(ra.N, ra.D);
  int64_t grid = (g.rows + 3) / 4;
  grid = grid < 1 ? 1 : (grid > 256 ? 256 : grid);
  const dim3 gd((unsigned)grid), wg(256);
  if (ra.E <= 8) {
    if (a.k <= 2) hipLaunchKernelGGL((k_route_dispatch_small<8, 2>), gd, wg, 0, s, ra, rs.S, a, g);
    else hipLaunchKernelGGL((k_route_dispatch_small<8, kMaxK>), gd, wg, 0, s, ra, rs.S, a, g);
  } else {
    if (a.k <= 2) hipLaunchKernelGGL((k_route_dispatch_small<16, 2>), gd, wg, 0, s, ra, rs.S, a, g);
    else hipLaunchKernelGGL((k_route_dispatch_small<16, kMaxK>), gd, wg, 0, s, ra, rs.S, a, g);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(k_gather<16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
