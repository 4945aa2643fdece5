// moe_internal.h: host-side launchers of the gfx950 kernels and the scratch layout.
// (Internal header of the HIP library; the public C ABI is include/moe.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kRouterTokens = 32;     // tokens per router partial-sum block (psum)
constexpr int kRouterTile = 256;      // tokens per split-K router workgroup (8 waves x 32)
constexpr int kRouterChunk = 64;      // K per pipeline step of the split-K router
constexpr int kDispatchTokens = 256;  // tokens per dispatch workgroup
constexpr int kSmallRows = 4096;       // most buffer rows of the fused one-launch dispatch
constexpr int kMaxE = 64;
constexpr int kMaxK = 8;
constexpr uint32_t kPsumMagic = 0x5053554du;  // marks valid router partial sums
// Marks token probabilities [N][E] left in the split-K partial region by the token-parallel
// router (the statistics then form the 32-token block sums themselves).
constexpr uint32_t kProbsMagic = 0x50524f42u;
constexpr int kTokRouterTokens = 64;  // most tokens of the token-parallel router
// Split-K partial tiles of the bf16 grouped GEMM: at most 256 workgroups, each holding
// 8 waves x 128 fp32 accumulators x 64 lanes.
constexpr size_t kGemmPartialUnits = 256;
constexpr size_t kGemmPartialBytes = kGemmPartialUnits * 8 * 128 * 64 * sizeof(float);
// After the partial tiles: the word that tells the fix-up kernel whether partials exist.
constexpr size_t kGemmFixupBytes = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Split-K router plan for bf16 x: `tiles` token tiles of kRouterTile tokens times S
// splits of D (Ks = D / S, a multiple of kRouterChunk), about 256 workgroups in all.
struct RouterSplit {
  int tiles, S, Ks;
};
#ifndef MOE_ROUTER_SMAX
#define MOE_ROUTER_SMAX 32
#endif
inline RouterSplit router_split(int64_t N, int64_t D) {
  RouterSplit r;
  r.tiles = (int)((N + kRouterTile - 1) / kRouterTile);
  const int chunks = (int)(D / kRouterChunk);
  int S = r.tiles >= 256 ? 1 : 256 / r.tiles;
  if (S > MOE_ROUTER_SMAX) S = MOE_ROUTER_SMAX;
  if (S > chunks) S = chunks;
  if (S < 1) S = 1;
  while (chunks % S != 0) --S;
  r.S = S;
  r.Ks = (int)(D / S);
  return r;
}
// Scratch (moe_scratch_size bytes) carved into regions, each 256-byte aligned:
//   header    : moe_stats (64 B) + magic word
//   psum      : fp32 [nblk_r][E]   per-router-block sums of the probabilities
//   blockcnt  : int32 [E][k][nblk_d] per-dispatch-block expert histogram of each slot
//               (token-major order: one segment [E][1][nblk_d] over all slots)
//   base      : int32 [E][k][nblk_d] exclusive scan of blockcnt in record order
//   tokdrop   : int32 [nblk_d]     tokens with every slot dropped, per block
//   load      : int32 [E]          copy of the pre-capacity histogram
//   partial   : fp32 split-K partial tiles of the bf16 grouped GEMM (bf16 layers only)
//   rpart     : fp32 [S][N][E] split-K partial router logits (bf16 layers only)
struct ScratchLayout {
  size_t header, psum, blockcnt, base, tokdrop, load, partial, rpart, total;
  int nblk_r, nblk_d;
};

inline ScratchLayout scratch_layout(int64_t N, int64_t D, int E, int k, bool bf16) {
  ScratchLayout s;
  s.nblk_r = (int)((N + kRouterTokens - 1) / kRouterTokens);
  s.nblk_d = (int)((N + kDispatchTokens - 1) / kDispatchTokens);
  size_t o = 0;
  s.header = o; o = align_up(o + 128, 256);
  s.psum = o; o = align_up(o + sizeof(float) * (size_t)s.nblk_r * E, 256);
  s.blockcnt = o; o = align_up(o + sizeof(int32_t) * (size_t)k * s.nblk_d * E, 256);
  s.base = o; o = align_up(o + sizeof(int32_t) * (size_t)k * s.nblk_d * E, 256);
  s.tokdrop = o; o = align_up(o + sizeof(int32_t) * (size_t)s.nblk_d, 256);
  s.load = o; o = align_up(o + sizeof(int32_t) * (size_t)E, 256);
  s.partial = o; o = align_up(o + (bf16 ? kGemmPartialBytes + kGemmFixupBytes : 0), 256);
  s.rpart = o; o = align_up(o + (bf16 ? sizeof(float) * (size_t)router_split(N, D).S * N * E : 0), 256);
  s.total = o;
  return s;
}

// ---- router -------------------------------------------------------------------------
struct RouterArgs {
  const void* x;          // [N,D] fp32 or bf16
  const float* w_r;       // [D,E]
  const float* bias;      // [E] or null
  const float* noise;     // [N,E] or null
  const float* logits_in; // [N,E] or null
  float* logits_out;      // [N,E] or null
  float* probs_out;       // [N,E] or null
  int32_t* topk_idx;      // [N,k]
  float* topk_gate;       // [N,k]
  float* psum;            // [nblk_r][E] or null
  uint32_t* psum_magic;   // or null
  float* rpart;           // [S][N][E] split-K partial logits (null: single-pass router)
  int64_t N;
  int D, E, k, mode;
  int noisy;  // MOE_SECOND_*: 1 = noise on slots >= 1, 2 = noise replaces the logits
};
hipError_t launch_router(const RouterArgs& a, bool bf16_x, hipStream_t s);
// Whether launch_router takes the token-parallel path for bf16 x with split-K scratch (and
// no given logits): batches of at most kTokRouterTokens tokens and at most 16 experts.
inline bool router_token_parallel(int64_t N, int E) { return N <= kTokRouterTokens && E <= 16; }
// Only the split-K logit kernel (bf16 x): partial logits [S][N][E] in a.rpart, S from
// router_split(N, D); the epilogue is left to the caller.
hipError_t launch_router_split(const RouterArgs& a, hipStream_t s);

// ---- dispatch -----------------------------------------------------------------------
struct DispatchArgs {
  const int32_t* topk_idx;  // [N,k]
  const float* topk_gate;   // [N,k]
  int32_t* blockcnt;        // scratch
  int32_t* base;            // scratch
  int32_t* tokdrop;         // scratch
  int32_t* load_copy;       // scratch
  int32_t* load;            // [E]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* row_of;          // [N,k]
  uint8_t* dropped;         // [N,k]
  float* gate_eff;          // [N,k]
  int32_t* token_of_row;    // [rows]
  int64_t N;
  int E, k, nblk;
  int64_t C;                // -1: no capacity
  int padded;
  int token_major;          // positions in token-major record order (else slot-major)
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

struct GatherArgs {
  const void* x;            // [N,D]
  int32_t* token_of_row;    // [rows] (padding rows set to -1 here)
  const int32_t* counts;    // [E]
  void* x_perm;             // [rows,D]
  int64_t rows, N;
  int D, elem_bytes;
  int64_t C;
  int padded;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_dispatch_small(const DispatchArgs& a, const GatherArgs& g, hipStream_t s);
// Router epilogue (from the split-K partial logits in ra.rpart) and dispatch in one launch:
// N <= kDispatchTokens, rows <= kSmallRows, E <= 16, no logits/probs outputs.
hipError_t launch_route_dispatch_small(const RouterArgs& ra, const DispatchArgs& a, const GatherArgs& g,
                                       hipStream_t s);

struct StatsArgs {
  const float* psum;
  const uint32_t* psum_magic;
  const float* probs;       // [N][E] token probabilities (token-parallel router), or null
  const int32_t* load;      // scratch copy
  const int32_t* tokdrop;
  void* out;                // moe_stats in the scratch header
  int64_t N, C;
  int E, k, nblk_r, nblk_d;
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t s);

// ---- expert FFN -----------------------------------------------------------------------
struct FfnArgs {
  const void* x_perm;       // [rows,D]
  const int32_t* offsets;   // [E+1]
  const int32_t* counts;    // [E]
  const void* w1;           // [E,D,F] (bf16 / fp32, or int8 when s1 is set)
  const void* w2;           // [E,D,F]
  const void* w3;           // [E,F,D]
  const float* s1;          // [E,F] int8 column scales of w1 (null: w1 in the layer dtype)
  const float* s2;          // [E,F]
  const float* s3;          // [E,D]
  void* h;                  // [rows,F]
  void* y_perm;             // [rows,D]
  int64_t rows;             // rows of the expert buffers
  int64_t max_rows_per_expert;  // host bound on counts[e] (N, or C when padded)
  int D, F, E, act;
  float* partial;           // scratch for split-K partial tiles (kGemmPartialBytes), then
                            // the fix-up word (kGemmFixupBytes)
  const int32_t* x_row_token;  // or null: x_perm is then x [N,D] and expert-buffer row r of
                               // the up-projection is x row x_row_token[r] (gathered rows)
};
// Gated up-projection (h) and down-projection (y_perm) of every expert's rows.
hipError_t launch_expert_up(const FfnArgs& a, bool bf16, hipStream_t s);
// True if the up-projection for these arguments can read its rows gathered from x
// (bf16 activations and weights, tiles of more than 64 rows).
bool expert_up_gathers(const FfnArgs& a, bool bf16);
hipError_t launch_expert_down(const FfnArgs& a, bool bf16, hipStream_t s);

// ---- combine --------------------------------------------------------------------------
struct CombineArgs {
  const void* y_perm;       // [rows,D]
  const int32_t* row_of;    // [N,k]
  const float* gate_eff;    // [N,k]
  void* y;                  // [N,D]
  int64_t N, rows;
  int D, k;
};
hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t s);

}  // namespace moe
