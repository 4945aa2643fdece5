// gemm_bf16.hip: bf16 grouped GEMMs of the expert FFN on gfx950 matrix cores.
//
// Method ("第 12 章 MoE：路由、专家与负载" §12.1 gated FFN f_e(x) = [SiLU(x W1_e) * (x W2_e)] W3_e
// with W1, W2 [D,F] and W3 [F,D]; "第 5 章 model.py 精读·中：MoE 路由与专家" §5.3.5 the same form
// with GELU, and §5.3.2 the expert weights stacked on a leading expert axis):
//   up   : h[r,:]      = act(x_perm[r,:] W1_e) * (x_perm[r,:] W2_e)
//   down : y_perm[r,:] = h[r,:] W3_e
// for the rows r of each expert e (rows [offsets[e], offsets[e] + counts[e])).
//
// Design.
//  * Work unit: a BM x (NB * BNF) output tile of one expert, computed by 8 waves. For
//    BM = 256 the waves form a 2 x 4 grid and each owns a 128-row block of fp32 MFMA
//    accumulators (128 per lane). The up projection has NB = 2: the W1 and W2 tiles of the
//    same columns sit side by side, so act(.) * (.) is formed in registers and h is stored
//    once in bf16.
//  * v_mfma_f32_32x32x16_bf16 with the operands swapped (weights as the first operand),
//    so each lane ends with 4 consecutive output columns of one row and stores 8 bytes.
//  * K loop over BK-wide slices in a ring of STAGES LDS buffers, filled by direct
//    global-to-LDS copies (global_load_lds_dwordx4) that need no staging registers. A (K
//    contiguous) is read with ds_read_b128; B (weights stored N contiguous) keeps its
//    natural layout and is turned into MFMA operands by the gfx950 transposing read
//    ds_read_b64_tr_b16 (ds_read_b64_tr_b8 plus an exact widening for int8 weights).
//    Both LDS tiles are unpadded and XOR-swizzled so these reads are bank-conflict free.
//    The bf16 256-row tiles split the 160 KB of LDS into two A slices and three B slices:
//    the A copies of slice kt + 1 go out after the barrier, those of B slice kt + 2 one
//    share after each 16-deep MFMA group of slice kt, so copy issue overlaps the MFMAs.
//  * Persistent, XCD-aware schedule: the grid is a multiple of 8 workgroups; workgroup b
//    runs on XCD b mod 8 and walks a contiguous eighth of the tile list, so the tiles
//    sharing one expert's activations and weight columns run concurrently inside one
//    XCD's L2. The last partial round is split along K; a fix-up kernel sums the pieces in
//    a fixed order. With at most 64 rows per expert (decode), 64-row tiles and stream-K
//    spread the weight stream evenly over all compute units.
//  * The only m-tile of an expert with fewer than BM rows runs a copy of the K loop in
//    which waves whose rows all lie past the expert's count skip their copies and MFMAs.
#include <atomic>
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;

constexpr int kXcds = 8;
constexpr int kSplitMax = 8;  // most K pieces of one tail tile

// Pipeline shape of the grouped GEMM: K slice per LDS stage and ring depth.
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
#ifndef MOE_GEMM_B3
#define MOE_GEMM_B3 1
#endif

__device__ __forceinline__ bf16x8 tr_read_b16x8(const bf16* q, int row_stride) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(q));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(q + 4 * row_stride));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef i32x2 __attribute__((address_space(3))) * lds_i32x2_ptr;

// gfx950 8-bit transposing LDS read: in each 16-lane group, result lane i gets byte i % 8
// of the 8 bytes addressed by source lanes 2 j + i / 8, j = 0..7. With source lane s
// pointing at row k0 + s / 2 and column half 8 (s % 2) of a 16-column segment, result
// lane i holds column i of the segment for rows k0 .. k0 + 7.
__device__ __forceinline__ i32x2 tr_read_b8x8(const void* q) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_ptr)(q));
}

// Eight int8 values (little-endian in two dwords) -> eight bf16, exactly: each byte is
// sign-extended and converted to fp32 in one instruction (a byte-select operand), and a
// byte permute takes the upper halves of two results as a bf16 pair (|v| <= 128 has at most
// 8 significant bits, so dropping the low 16 bits of the fp32 value is exact): 1.5
// instructions per weight.
__device__ __forceinline__ bf16x8 i8x8_to_bf16(i32x2 r) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const float f0 = (float)(int32_t)(int8_t)(r[h] >> (16 * pr));
      const float f1 = (float)(int32_t)(int8_t)(r[h] >> (16 * pr + 8));
      o[2 * h + pr] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    }
  }
  return __builtin_bit_cast(bf16x8, o);
}

// Chunk swizzle of int8 B rows with CPR 16-byte chunks per row (8 or 16).
template <int CPR>
__device__ __forceinline__ int q8_swz(int row) {
  static_assert(CPR == 8 || CPR == 16, "int8 B rows of 128 or 256 bytes");
  return CPR == 8 ? 2 * ((row >> 1) & 3) : 2 * (row & 7);
}

// Direct-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes land
// at LDS byte address lds_addr + 16 l; lds_addr is wave-uniform and goes through M0.
// Written as inline asm so the compiler does not treat the in-flight copy as a pending
// write to every LDS location (it would then wait for all copies before each LDS read);
// completion is tracked explicitly with wait_vmcnt. The instruction has no destination
// register, and the leading s_nop covers the M0-write to LDS-DMA hazard.
__device__ __forceinline__ void load_lds16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// Waits until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads() (the fence would wait for
// every copy in flight). Visibility is explicit: each wave waits for its own copies of a
// slice before the barrier, and for its own LDS reads (lgkmcnt(0)) so that no read of a
// stage is still pending when another wave's copy refills that stage after the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const bf16* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) bf16*)p);
}

// Waits until this wave's copies of the slice `ahead` slices before the newest issued
// one have landed (each slice is LOADS copies per wave).
template <int LOADS>
__device__ __forceinline__ void wait_for_slice(int ahead) {
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<LOADS>(); break;
    case 2: wait_vmcnt<2 * LOADS>(); break;
    case 3: wait_vmcnt<3 * LOADS>(); break;
    case 4: wait_vmcnt<(4 * LOADS < 63 ? 4 * LOADS : 0)>(); break;
    case 5: wait_vmcnt<(5 * LOADS < 63 ? 5 * LOADS : 0)>(); break;
    default: wait_vmcnt<(6 * LOADS < 63 ? 6 * LOADS : 0)>(); break;
  }
}

// Epilogue of a tile: act(acc W1) * (acc W2) for the gated up-projection (NB = 2), the
// plain product otherwise, rounded once to bf16. With the operands swapped, accumulator
// element r of a lane holds row lane % 32 and column 8 (r / 4) + 4 (lane / 32) + r % 4
// of its 32 x 32 block, so each lane stores 4 consecutive bf16 (8 bytes).
// Output values of 4 consecutive columns (col .. col + 3 of the tile) from the raw
// accumulators a0 (B0) and a1 (B1): act(a0) * a1 for the gated up-projection, a0 otherwise,
// each first multiplied by its column scale when the weights are int8.
template <int NB, int ACT, bool Q8>
__device__ __forceinline__ bf16x4 epilogue4(const GemmParams& p, const Tile& tl, int col, f32x4 a0, f32x4 a1) {
  if constexpr (Q8) {
    const int64_t sc = (int64_t)tl.e * p.N + tl.n0 + col;
    a0 *= *reinterpret_cast<const f32x4*>(p.S0 + sc);
    if constexpr (NB == 2) a1 *= *reinterpret_cast<const f32x4*>(p.S1 + sc);
  }
  bf16x4 o;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v;
    if constexpr (NB == 2) v = activate<ACT>(a0[u]) * a1[u];
    else v = a0[u];
    o[u] = (bf16)v;
  }
  return o;
}

template <int NB, int ACT, int TM, int TN, int WM, int WN, bool Q8>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NB][TM][TN], const Tile& tl, const GemmParams& p,
                                           int wm, int wn, int lane) {
  const int N = p.N;
  bf16* Cg = reinterpret_cast<bf16*>(p.C) + tl.row_base * N + tl.n0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * WM + 32 * i + (lane & 31);
    if (row >= tl.mcount) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * WN + 32 * j + 8 * q + 4 * (lane >> 5);
        f32x4 a0, a1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a0[u] = acc[0][i][j][4 * q + u];
          a1[u] = acc[NB - 1][i][j][4 * q + u];
        }
        *reinterpret_cast<bf16x4*>(Cg + (int64_t)row * N + col) = epilogue4<NB, ACT, Q8>(p, tl, col, a0, a1);
      }
  }
}

// Stream-K range of workgroup w over the W = tiles * nk (tile, K slice) work items, and
// the workgroup that owns work item s.
__device__ __forceinline__ int64_t sk_begin(int64_t w, int64_t W, int64_t G) { return w * W / G; }
__device__ __forceinline__ int64_t sk_owner(int64_t s, int64_t W, int64_t G) { return ((s + 1) * G - 1) / W; }

// Stream-K schedule over G workgroups. All T tiles run whole (tile L on workgroup L % Gd,
// the other workgroups idle) when they fit in one round on Gd = T >= 5/8 G workgroups, or
// in r = ceil(T / G) rounds on Gd = ceil(T / r) >= 7/8 G: that many compute units already
// saturate HBM with the weight stream, and no partial tiles or fix-up work arise (measured
// on the decode shapes: one round on 168 workgroups beats stream-K on 256, two rounds on
// 168 do not, since a workgroup then has to stream ~40% faster). Otherwise the first
// dp = (T / G) G tiles run whole, one per workgroup per round, and the remaining R = T - dp
// tiles are cut into equal (tile, K slice) ranges, one per workgroup, so every workgroup
// streams the same number of K slices. When R <= G / 2 and R floor(G / R) >= 7/8 G, only
// g = R floor(G / R) workgroups take ranges: each range is then a 1 / floor(G / R) piece of
// one tile, so no range spans two tiles and a tile leaves floor(G / R) partials instead of
// up to G / R + 1 (decode down-projection, 48 tiles of 224 K slices: 240 workgroups, GEMM
// 67.1 + fix-up 8.9 us against 69.7 + 10.3 us on 256; int8 weights 45.7 + 8.9 against
// 47.6 + 10.0 us). The other g .. G - 1 workgroups run only their whole tiles.
#ifndef MOE_SK_WHOLE
#define MOE_SK_WHOLE 1
#endif
struct SkPlan {
  int dp;      // tiles run whole
  int64_t W;   // stream-K work items: (T - dp) * nk
  int stride;  // workgroups running the whole tiles
  int g;       // workgroups that take the stream-K ranges (workgroups 0 .. g - 1)
};
__device__ __forceinline__ SkPlan sk_plan(int T, int G, int nk) {
  SkPlan s;
  const int r = (T + G - 1) / G;
  const int gd = r > 0 ? (T + r - 1) / r : 0;
  if (MOE_SK_WHOLE && ((r == 1 && 8 * T >= 5 * G) || 8 * gd >= 7 * G)) {
    s.dp = T;
    s.W = 0;
    s.stride = gd;
    s.g = G;
    return s;
  }
  s.dp = T / G * G;
  s.W = (int64_t)(T - s.dp) * nk;
  s.stride = G;
  s.g = G;
  const int R = T - s.dp, P = R > 0 ? G / R : 0;
  if (P >= 2 && 8 * R * P >= 7 * G) s.g = R * P;
  return s;
}

// fp32 partial tiles. A slot holds one workgroup's raw accumulators of one tile as 16-byte
// groups: group g (of NACC / 4 per lane) of wave w, lane l at float4 index
// ((slot * 8 + w) * NACC / 4 + g) * 64 + l, with g = ((m * TM + i) * TN + j) * 4 + q
// holding accumulator elements 4q .. 4q + 3 of block (m, i, j).
// Wave grid of a workgroup (8 waves): 2 x 4 (rows x columns), or 1 x 8 for 64 x 256 tiles
// of int8 weights, where every wave then converts distinct weight columns.
template <int BM, int BNF, bool Q8>
struct WaveGrid {
  static constexpr int WGM = (Q8 && BM == 64 && BNF == 256) ? 1 : 2;
  static constexpr int WGN = 8 / WGM;
};

template <int BM, int BNF, int NB, bool Q8 = false>
struct Frag {
  static constexpr int WGN = WaveGrid<BM, BNF, Q8>::WGN;
  static constexpr int WM = BM / WaveGrid<BM, BNF, Q8>::WGM, WN = BNF / WGN, TM = WM / 32, TN = WN / 32;
  static constexpr int NACC = NB * TM * TN * 16;
  static constexpr int G4 = TM * TN * 4;       // 16-byte groups per matrix per lane
  static constexpr int ITEMS = 8 * G4 * 64;    // fix-up threads per tile
};

template <int BM, int BNF, int NB, bool Q8>
__device__ __forceinline__ f32x4* slot_base(const GemmParams& p, int64_t slot, int wid) {
  return reinterpret_cast<f32x4*>(p.partial) + (slot * 8 + wid) * (Frag<BM, BNF, NB, Q8>::NACC / 4) * 64;
}

// Threads per fix-up workgroup (the grid-stride loops below assume it).
constexpr int kFixupThreads = 256;

// Fix-up thread `it` of a tile: sums the 16-byte groups (one per matrix) of the slots that
// next_slot() yields, in order, applies the epilogue and stores 4 bf16 of one row.
template <int BM, int BNF, int NB, int ACT, bool Q8, typename Slots>
__device__ __forceinline__ void fixup_item(const GemmParams& p, const Tile& tl, int it, Slots next_slot) {
  using FR = Frag<BM, BNF, NB, Q8>;
  const int w = it / (FR::G4 * 64), rem = it % (FR::G4 * 64);
  const int g = rem / 64, lane = rem % 64;
  const int q = g % 4, ij = g / 4, i = ij / FR::TN, j = ij % FR::TN;
  const int row = (w / FR::WGN) * FR::WM + 32 * i + (lane & 31);
  if (row >= tl.mcount) return;  // past the expert's count: no partials stored
  f32x4 acc[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t slot;
  while (next_slot(slot)) {
    const f32x4* P = slot_base<BM, BNF, NB, Q8>(p, slot, w) + lane;
#pragma unroll
    for (int m = 0; m < NB; ++m) acc[m] += P[(m * FR::G4 + g) * 64];
  }
  const int col = (w % FR::WGN) * FR::WN + 32 * j + 8 * q + 4 * (lane >> 5);
  bf16* C = reinterpret_cast<bf16*>(p.C) + (tl.row_base + row) * p.N + tl.n0 + col;
  *reinterpret_cast<bf16x4*>(C) = epilogue4<NB, ACT, Q8>(p, tl, col, acc[0], acc[NB - 1]);
}

// Whether a launch leaves partials for its fix-up kernel: a persistent launch of gd
// workgroups when some XCD share splits its tail round along K, a stream-K launch when its
// ranges cut tiles at all (conservative: W > 0). Wave-wide (tile_scan).
template <int BM, int BK>
__device__ __forceinline__ bool persistent_splits(const GemmParams& p, int gd) {
  const int nslot = gd / kXcds;
  if (p.partial == nullptr || nslot <= 0) return false;
  const TileScan ts = tile_scan<BM>(p);
  bool any = false;
  for (int x = 0; x < kXcds; ++x) any = any || xcd_share(ts.total, x, kXcds, nslot, p.K / BK, p).S > 1;
  return any;
}
template <int BM, int BK>
__device__ __forceinline__ bool streamk_partials(const GemmParams& p, int gd) {
  return gd > 0 && sk_plan(tile_scan<BM>(p).total, gd, p.K / BK).W > 0;
}
// Run by wave 0 of workgroup 0 at the start of a launch: the fix-up word for this launch
// (the previous launch's fix-up has finished: same stream).
__device__ __forceinline__ void set_fixup(const GemmParams& p, bool need) {
  if (p.fixup != nullptr && lane_id() == 0) *p.fixup = need ? 1u : 0u;
}
// A fix-up kernel's first step: nothing to do when the GEMM launch left no partials.
__device__ __forceinline__ bool fixup_idle(const GemmParams& p) { return p.fixup != nullptr && *p.fixup == 0u; }

// STREAMK = false: persistent full tiles per XCD share, tail round split along K.
// STREAMK = true : stream-K; the (tile, K slice) list is cut into equal contiguous ranges,
//                  one per workgroup; a tile cut by a range boundary leaves fp32 partials
//                  (slot 2w for the workgroup's first tile, 2w + 1 for its last).
// LDS ring of one tile configuration, in bf16 elements.
template <int BM, int BNF, int NB, int BK, int STAGES, bool STREAMK, bool Q8>
struct Ring {
  static constexpr int A_EL = BM * BK, B_BYTES = BK * BNF * (Q8 ? 1 : 2);
  static constexpr int STAGE = A_EL + NB * B_BYTES / 2;
  static constexpr bool B3 = MOE_GEMM_B3 && !STREAMK && !Q8 && STAGES == 2;
  static constexpr int EL = B3 ? 2 * A_EL + 3 * (NB * B_BYTES / 2) : STAGES * STAGE;
};

template <int BM, int BNF, int NB, int ACT, int BK, int STAGES, bool STREAMK, bool Q8, bool GA = false>
__device__ __forceinline__ void gemm_tiles(const GemmParams& p, bf16* ring, const int bx, const int gd) {
  // bx, gd: this workgroup's index among the gd workgroups that share the tile list
  // (blockIdx.x and gridDim.x, or one part of the grid of a mixed-height launch; gd % 8 == 0).
  // GA: gathered A rows (p.row_token).
  // BK: K slice per pipeline stage; STAGES: LDS ring depth (STAGES-1 slices in flight).
  // Q8: B0/B1 are int8 with per-column scales S0/S1 (weight-only 8-bit experts).
  constexpr int WB = Q8 ? 1 : 2;            // bytes per B element
  constexpr int WGN = WaveGrid<BM, BNF, Q8>::WGN;
  constexpr int WM = BM / WaveGrid<BM, BNF, Q8>::WGM, WN = BNF / WGN;  // wave tile per matrix
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_EL = BM * BK, B_BYTES = BK * BNF * WB;
  constexpr int STAGE = A_EL + NB * B_BYTES / 2;    // bf16 elements per ring stage
  constexpr int A_COPIES = A_EL * 2 / 1024;         // 1 KB copies of one A slice
  constexpr int A_CP = A_COPIES >= 8 ? A_COPIES / 8 : 1;  // 1 KB copies per copying wave per slice
  constexpr int A_WAVES = A_COPIES / A_CP;           // waves copying A (all 8 but for small slices)
  constexpr int B_CPM = B_BYTES / 1024;             // 1 KB copies per matrix per slice
  constexpr int B_CP = NB * B_CPM / 8;              // B copies per wave per slice
  constexpr int LOADS = A_CP + B_CP;
  constexpr int B_RPC = 1024 / (BNF * WB);          // B rows per copy
  constexpr int B_CPR = BNF * WB / 16;              // 16-byte chunks per B row
  constexpr int A_CPR = BK / 8;                     // 16-byte chunks per A row
  constexpr int A_RPB = 128 / BK;                   // A rows per 256 bytes (64 banks)
  constexpr int A_RPC = 512 / BK;                   // A rows per 1 KB copy
  static_assert((BM == 256 || BM == 64) && (BNF == 128 || BNF == 256) && (BK == 32 || BK == 64), "tile shape");
  static_assert(!Q8 || BK == 64, "int8 tiles: 64-deep slices");
  static_assert(STAGES >= 2 && STAGES <= 8 && STAGES * STAGE * 2 <= 160 * 1024, "LDS ring");
  static_assert(A_COPIES >= 1 && A_CP * A_WAVES == A_COPIES && B_CP >= 1 && TM >= 1 && TN >= 1 &&
                (NB * B_CPM) % 8 == 0, "tile shape");
  static_assert(A_WAVES == 8 || STREAMK, "small A slices: stream-K tiles only");
  // Split ring (persistent bf16 tiles with 2 stages): A slices double-buffered, B slices
  // triple-buffered, and the copies of B slice kt + 2 spread between the MFMA groups of
  // slice kt instead of issued in one burst after the barrier.
  constexpr bool B3 = MOE_GEMM_B3 && !STREAMK && !Q8 && STAGES == 2;
  constexpr int B_EL = NB * B_BYTES / 2;  // bf16 elements of one B slice (all matrices)
  constexpr int RING_EL = B3 ? 2 * A_EL + 3 * B_EL : STAGES * STAGE;
  static_assert(RING_EL * 2 <= 160 * 1024, "LDS ring");
  static_assert(RING_EL == Ring<BM, BNF, NB, BK, STAGES, STREAMK, Q8>::EL, "LDS ring size");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int wm = wid / WGN, wn = wid % WGN;
  const int K = p.K, N = p.N;
  const int nk = K / BK;

  const TileScan ts = tile_scan<BM>(p);
  const int xcd = bx % kXcds;
  const int slot = bx / kXcds;
  const int nslot = gd / kXcds;
  const XcdShare sh = xcd_share(ts.total, xcd, kXcds, nslot, nk, p);

  // LDS layouts (no padding; 16-byte chunks XOR-swizzled so the MFMA operand reads are
  // bank-conflict free):
  //   A [BM][BK]: row r, logical chunk c (8 elements) at physical chunk c ^ f(r),
  //               f(r) = (r / A_RPB) % A_CPR, so 16 consecutive rows hit 16 bank groups.
  //   B [BK][BNF]: row k, logical 32-byte segment g at physical segment g ^ (2 (k % 4)).
  //   B int8 [BK][BNF]: row k (BNF bytes), logical 16-byte chunk c at physical chunk
  //               c ^ q8_swz(k), q8_swz(k) = 2 ((k / 2) % 4) for 128-byte rows and 2 (k % 8)
  //               for 256-byte rows: the 8 rows x 2 chunks of one 8-bit transposing read
  //               by two 16-lane groups then fill 16 distinct bank groups.
  // Fragment addresses (constant per lane):
  //   A: lane -> row (lane % 32) of each 32-row block, k chunk 2 kk + lane / 32.
  //   B: transposing read; 16-lane group G -> column half (G & 1), k-half (G >> 1); lane s
  //      of the group supplies row s / 4 and columns 4 (s % 4) .. +3 of a 4 x 16 block.
  //   B int8: 8-bit transposing read; group G -> columns 16 (G & 1) .. +15 of the 32-column
  //      block, rows 8 (G >> 1) .. +7; lane s supplies row s / 2, column half s % 2.
  const int a_row = wm * WM + (lane & 31);
  const int a_swz = ((lane & 31) / A_RPB) % A_CPR;
  const int G = lane >> 4, s16 = lane & 15;
  const int b_row = 8 * (G >> 1) + (s16 >> 2);
  const int b_swz = 2 * (s16 >> 2);
  const int b_seg = (wn * WN) / 16 + (G & 1);
  const int b_in = 4 * (s16 & 3);

  // Copy coordinates. A copy c covers rows A_RPC c ..: lane -> row A_RPC c + lane / A_CPR
  // and physical chunk lane % A_CPR, which holds logical chunk (lane % A_CPR) ^ f(row).
  // B copy c (matrix c / B_CPM) covers rows B_RPC (c % B_CPM) ..: lane -> row + lane /
  // B_CPR and physical chunk pc = lane % B_CPR, holding logical chunk 2 ((pc / 2) ^ h) +
  // (pc & 1) with h = 2 (row % 4).
  const int ring_addr = (int)lds_addr_of(ring);

  // Work units of this workgroup. Persistent: its full-K tiles of each round, then (if
  // any) one K piece of a tail tile. Stream-K: every tile its range touches.
  int units, sk_t0 = 0, dp_rounds = 0;
  int64_t sk_s0 = 0, sk_s1 = 0;
  SkPlan sk{0, 0, 1, 1};
  if constexpr (STREAMK) {
    sk = sk_plan(ts.total, gd, nk);
    const int b = bx;
    dp_rounds = b < min(sk.dp, sk.stride) ? (sk.dp - b + sk.stride - 1) / sk.stride : 0;
    if (bx < sk.g) {  // workgroups past sk.g take no stream-K range
      sk_s0 = sk_begin(bx, sk.W, sk.g);
      sk_s1 = sk_begin(bx + 1, sk.W, sk.g);
    }
    sk_t0 = (int)(sk_s0 / nk);
    units = dp_rounds + (sk_s1 > sk_s0 ? (int)((sk_s1 - 1) / nk) - sk_t0 + 1 : 0);
  } else {
    units = sh.rounds + (slot < sh.tail * sh.S ? 1 : 0);
  }
  // K range, tile index and partial slot of unit u.
  auto unit_of = [&](int u, int& L, int& kb, int& ke, int& pslot) {
    kb = 0;
    ke = nk;
    pslot = -1;
    if constexpr (STREAMK) {
      if (u < dp_rounds) {
        L = bx + u * sk.stride;
      } else {
        const int ls = sk_t0 + (u - dp_rounds);  // tile index within the stream-K tiles
        const int64_t base = (int64_t)ls * nk;
        kb = (int)(max(sk_s0, base) - base);
        ke = (int)(min(sk_s1, base + nk) - base);
        if (kb != 0 || ke != nk) pslot = 2 * bx + (u == dp_rounds ? 0 : 1);
        L = sk.dp + ls;
      }
    } else if (u < sh.rounds) {
      L = sh.lo + slot + u * nslot;
    } else {
      const int i = slot % sh.tail, piece = slot / sh.tail;
      L = sh.lo + sh.rounds * nslot + i;
      kb = piece * nk / sh.S;
      ke = (piece + 1) * nk / sh.S;
      if (sh.S > 1) pslot = xcd * nslot + slot;
    }
  };
  // Gathered A (p.row_token): A row r of the product is row
  // row_token[r] of p.A. Lane's A copy q covers row A_RPC (A_CP wid + q) + lane / A_CPR of
  // the tile; its token is read one tile ahead, before the epilogue of the previous tile.
  auto load_tokens = [&](const Tile& t, int (&tk)[A_CP]) {
#pragma unroll
    for (int q = 0; q < A_CP; ++q) {
      const int row = A_RPC * (A_CP * wid + q) + lane / A_CPR;
      tk[q] = p.row_token[t.row_base + min(row, t.mcount - 1)];
    }
  };
  int tok_next[A_CP];
  int tok_unit = -1;  // unit whose tokens tok_next holds
  for (int u = 0; u < units; ++u) {
    int L, kb, ke, pslot;
    unit_of(u, L, kb, ke, pslot);
    Tile tl;
    if (!tile_of<BM, BNF>(p, ts, L, tl)) continue;

    const bf16* Ag = reinterpret_cast<const bf16*>(p.A) + tl.row_base * K;
    const int64_t boff = (int64_t)tl.e * K * N + tl.n0;
    const int mlast = tl.mcount - 1;  // rows past the expert's count re-read a valid row

    const bf16* a_src[A_CP];
    if constexpr (GA) {
      int tok[A_CP];
      if (tok_unit == u) {
#pragma unroll
        for (int q = 0; q < A_CP; ++q) tok[q] = tok_next[q];
      } else {
        load_tokens(tl, tok);
      }
#pragma unroll
      for (int q = 0; q < A_CP; ++q) {
        const int row = A_RPC * (A_CP * wid + q) + lane / A_CPR;
        const int lc = (lane % A_CPR) ^ ((row / A_RPB) % A_CPR);
        a_src[q] = reinterpret_cast<const bf16*>(p.A) + (int64_t)tok[q] * K + 8 * lc;
      }
    } else {
#pragma unroll
      for (int q = 0; q < A_CP; ++q) {
        const int c = A_CP * wid + q;
        const int row = A_RPC * c + lane / A_CPR;
        const int lc = (lane % A_CPR) ^ ((row / A_RPB) % A_CPR);
        a_src[q] = Ag + (int64_t)min(row, mlast) * K + 8 * lc;
      }
    }
    const char* b_src[B_CP];  // byte addresses
#pragma unroll
    for (int q = 0; q < B_CP; ++q) {
      const int c = B_CP * wid + q;
      const int m = c / B_CPM;
      const int row = B_RPC * (c % B_CPM) + lane / B_CPR;
      const int pc = lane % B_CPR;
      int lc;
      if constexpr (Q8) lc = pc ^ q8_swz<B_CPR>(row);
      else lc = 2 * ((pc >> 1) ^ (2 * (row & 3))) + (pc & 1);
      const char* Bm = reinterpret_cast<const char*>(m == 0 ? p.B0 : p.B1);
      b_src[q] = Bm + (boff + (int64_t)row * N) * WB + 16 * lc;
    }

    const int nku = ke - kb;  // K slices of this unit
    auto issue_slice = [&](int kt, bool with_a) {
      const int k0 = (kb + kt) * BK;
      const int base = ring_addr + (kt % STAGES) * STAGE * 2;
      if (with_a) {
#pragma unroll
        for (int q = 0; q < A_CP; ++q) load_lds16(a_src[q] + k0, (uint32_t)uniform(base + (A_CP * wid + q) * 1024));
      }
#pragma unroll
      for (int q = 0; q < B_CP; ++q)
        load_lds16(b_src[q] + (int64_t)k0 * N * WB, (uint32_t)uniform(base + A_EL * 2 + (B_CP * wid + q) * 1024));
    };
    // split ring: A slice kt in A slot kt % 2, B slice kt in B slot kt % 3
    auto issue_a = [&](int kt) {
      const int k0 = (kb + kt) * BK;
      const int base = ring_addr + (kt % 2) * A_EL * 2;
#pragma unroll
      for (int q = 0; q < A_CP; ++q) load_lds16(a_src[q] + k0, (uint32_t)uniform(base + (A_CP * wid + q) * 1024));
    };
    // copies q of B slice kt with q0 <= q < q1 (q0, q1 compile-time after unrolling)
    auto issue_b = [&](int kt, int q0, int q1) {
      const int k0 = (kb + kt) * BK;
      const int base = ring_addr + 2 * A_EL * 2 + (kt % 3) * B_EL * 2;
#pragma unroll
      for (int q = 0; q < B_CP; ++q)
        if (q >= q0 && q < q1)
          load_lds16(b_src[q] + (int64_t)k0 * N * WB, (uint32_t)uniform(base + (B_CP * wid + q) * 1024));
    };

    f32x16 acc[NB][TM][TN];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

    // K loop, in two copies. The plain one serves every tile but one kind: the only m-tile
    // of an expert with fewer than BM rows (common with many small experts). In its copy, a
    // wave whose A copies cover no valid row skips them and a wave whose accumulator rows
    // all lie past the count skips its LDS reads and MFMAs; the stale LDS rows feed only
    // accumulator rows that are never stored.
    auto k_loop = [&](auto lone_tile) {
      constexpr bool LONE = decltype(lone_tile)::value;
      const bool a_live = wid < A_WAVES && (!LONE || A_RPC * A_CP * wid < tl.mcount);
      const bool c_live = !LONE || wm * WM < tl.mcount;
    if constexpr (B3) {
      // Issue order per wave: A0, B0, B1 | A1, B2 | A2, B3 | ... (iteration kt issues A kt+1
      // after its barrier and B kt+2 between its MFMA groups), so when iteration kt starts
      // at most the copies of B kt+1 may still be outstanding after A kt and B kt.
      constexpr int GROUPS = BK / 16;  // MFMA groups (16-deep K steps); B copies split over them
      if (a_live) issue_a(0);
      issue_b(0, 0, B_CP);
      if (nku > 1) issue_b(1, 0, B_CP);
      for (int kt = 0; kt < nku; ++kt) {
        if (kt + 1 < nku) wait_vmcnt<B_CP>();
        else wait_vmcnt<0>();
        barrier_no_fence();  // A kt and B kt visible to every wave; slice kt-1 fully consumed
        if (a_live && kt + 1 < nku) issue_a(kt + 1);
        const bool b2 = kt + 2 < nku;
        if (!c_live) {
          if (b2) issue_b(kt + 2, 0, B_CP);
          continue;
        }
        const bf16* As = ring + (kt % 2) * A_EL;
        const bf16* Bs = ring + 2 * A_EL + (kt % 3) * B_EL;
        // fragments of one 16-deep group, read one group ahead (two groups live)
        bf16x8 af[2][TM], bfr[2][NB][TN];
        auto load_group = [&](int kk, int buf) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
            af[buf][i] = *reinterpret_cast<const bf16x8*>(As + (a_row + 32 * i) * BK + 8 * ((2 * kk + (lane >> 5)) ^ a_swz));
#pragma unroll
          for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              bfr[buf][m][j] = tr_read_b16x8(Bs + m * (B_BYTES / 2) + (kk * 16 + b_row) * BNF +
                                                 16 * ((b_seg + 2 * j) ^ b_swz) + b_in, BNF);
        };
        load_group(0, 0);
#pragma unroll
        for (int kk = 0; kk < GROUPS; ++kk) {
          if (kk + 1 < GROUPS) load_group(kk + 1, (kk + 1) & 1);
#pragma unroll
          for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int i = 0; i < TM; ++i)
                acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][m][j], af[kk & 1][i], acc[m][i][j], 0, 0, 0);
          // this group's share of the copies of B slice kt + 2, kept between the MFMA groups
          const int q0 = kk * B_CP / GROUPS, q1 = (kk + 1) * B_CP / GROUPS;  // unrolled: constants
          if (q1 > q0 && b2) {
            __builtin_amdgcn_sched_barrier(0);
            issue_b(kt + 2, q0, q1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nku) issue_slice(st, a_live);

    for (int kt = 0; kt < nku; ++kt) {
      // Slice kt has landed once at most (slices issued after it) * (copies per slice) remain.
      if (a_live) wait_for_slice<LOADS>(min(STAGES - 2, nku - 1 - kt));
      else wait_for_slice<B_CP>(min(STAGES - 2, nku - 1 - kt));
      barrier_no_fence();  // slice kt visible to every wave; slice kt-1 fully consumed
      if (kt + STAGES - 1 < nku) issue_slice(kt + STAGES - 1, a_live);
      if (!c_live) continue;

      const bf16* As = ring + (kt % STAGES) * STAGE;
      bf16x8 af[BK / 16][TM], bfr[BK / 16][NB][TN];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[kk][i] = *reinterpret_cast<const bf16x8*>(As + (a_row + 32 * i) * BK + 8 * ((2 * kk + (lane >> 5)) ^ a_swz));
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (Q8) {
              const char* Bs = reinterpret_cast<const char*>(As + A_EL) + m * B_BYTES;
              const int row = kk * 16 + 8 * (G >> 1) + (s16 >> 1);
              const int chunk = (wn * WN + 32 * j) / 16 + (G & 1);
              bfr[kk][m][j] =
                  i8x8_to_bf16(tr_read_b8x8(Bs + row * BNF + 16 * (chunk ^ q8_swz<B_CPR>(row)) + 8 * (s16 & 1)));
            } else {
              bfr[kk][m][j] = tr_read_b16x8(As + A_EL + m * (B_BYTES / 2) + (kk * 16 + b_row) * BNF +
                                                16 * ((b_seg + 2 * j) ^ b_swz) + b_in, BNF);
            }
          }
      }
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
              acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk][m][j], af[kk][i], acc[m][i][j], 0, 0, 0);
    }
    };
    if constexpr (STREAMK) {
      k_loop(std::false_type{});
    } else {
      if (tl.m0 == 0 && tl.mcount < BM) k_loop(std::true_type{});
      else k_loop(std::false_type{});
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave done reading the ring before the next tile refills it
    if constexpr (GA) {
      // tokens of the next unit that has a tile, requested before this tile's stores
      for (int un = u + 1; un < units; ++un) {
        int L2, kb2, ke2, ps2;
        unit_of(un, L2, kb2, ke2, ps2);
        Tile t2;
        if (!tile_of<BM, BNF>(p, ts, L2, t2)) continue;
        load_tokens(t2, tok_next);
        tok_unit = un;
        break;
      }
    }

    if (pslot >= 0) {
      // A K piece of a tile: keep the raw fp32 accumulators of the rows below the expert's
      // count for the fix-up (the fix-up reads no others).
      f32x4* P = slot_base<BM, BNF, NB, Q8>(p, pslot, wid) + lane;
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            if (wm * WM + 32 * i + (lane & 31) < tl.mcount)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              P[(((m * TM + i) * TN + j) * 4 + q) * 64] =
                  f32x4{acc[m][i][j][4 * q], acc[m][i][j][4 * q + 1], acc[m][i][j][4 * q + 2], acc[m][i][j][4 * q + 3]};
    } else {
      store_tile<NB, ACT, TM, TN, WM, WN, Q8>(acc, tl, p, wm, wn, lane);
    }
  }
}

template <int BM, int BNF, int NB, int ACT, int BK, int STAGES, bool STREAMK, bool Q8, bool GA = false>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 ring[Ring<BM, BNF, NB, BK, STAGES, STREAMK, Q8>::EL];
  if (blockIdx.x == 0 && threadIdx.x < 64) {  // before the tiles, so none of it stays live across them
    if constexpr (STREAMK) set_fixup(p, streamk_partials<BM, BK>(p, gridDim.x));
    else set_fixup(p, persistent_splits<BM, BK>(p, gridDim.x));
  }
  gemm_tiles<BM, BNF, NB, ACT, BK, STAGES, STREAMK, Q8, GA>(p, ring, blockIdx.x, gridDim.x);
}

// Skinny gated up-projection (every expert at most 64 rows) with two tile widths in one
// launch, chosen on the device from counts[]: 64 x (2 x 256) tiles (32-deep slices, four
// stages) when they fill one round of whole tiles (or several rounds on >= 7/8 of the
// workgroups) and 64 x (2 x 128) tiles would not, since their stream-K remainder then
// needs partials and a fix-up; 64 x (2 x 128) tiles (64-deep slices) otherwise. A whole tile
// of either width forms each output as one fp32 sum over K in the same order.
// p describes the narrow tiles (n_tiles = N / 128); N % 256 == 0.
constexpr int kSkinnyRows64 = 64;
__device__ __forceinline__ bool skinny_wide(const GemmParams& p, int grid) {
  const TileScan ts = tile_scan<kSkinnyRows64>(p);  // narrow tiles
  const SkPlan wide = sk_plan(ts.total / 2, grid, 1), narrow = sk_plan(ts.total, grid, 1);
  return wide.W == 0 && narrow.W != 0;
}

#ifndef MOE_DUAL_BK
#define MOE_DUAL_BK 32
#endif
#ifndef MOE_DUAL_STAGES
#define MOE_DUAL_STAGES 4
#endif
template <int ACT>
__global__ __launch_bounds__(512, 1) void k_gemm_skinny_dual(const GemmParams p) {
  constexpr int EL_N = Ring<64, 128, 2, 64, 4, true, false>::EL;
  constexpr int EL_W = Ring<64, 256, 2, MOE_DUAL_BK, MOE_DUAL_STAGES, true, false>::EL;
  __shared__ __attribute__((aligned(1024))) bf16 ring[EL_N > EL_W ? EL_N : EL_W];
  const bool wide = skinny_wide(p, gridDim.x);
  if (blockIdx.x == 0 && threadIdx.x < 64) set_fixup(p, !wide && streamk_partials<64, 64>(p, gridDim.x));
  if (wide) {
    GemmParams q = p;
    q.n_tiles = p.N / 256;
    gemm_tiles<64, 256, 2, ACT, MOE_DUAL_BK, MOE_DUAL_STAGES, true, false>(q, ring, blockIdx.x, gridDim.x);
  } else {
    gemm_tiles<64, 128, 2, ACT, 64, 4, true, false>(p, ring, blockIdx.x, gridDim.x);
  }
}

// Fix-up of the tail split: sums the K pieces of every split tail tile in piece order and
// stores the tiles. Grid-stride over (tail tile, fix-up thread); the tail tiles of the XCD
// shares are numbered in XCD order. Repeats the GEMM's schedule arithmetic from counts[]
// so both kernels agree on the split. Every wave handles 64 consecutive threads of one
// tile (ITEMS is a multiple of 64), so the tile lookup stays wave-uniform.
template <int BM, int BNF, int NB, int ACT, int BK, bool Q8>
__device__ __forceinline__ void tail_reduce(const GemmParams& p, const int nslot) {
  using FR = Frag<BM, BNF, NB, Q8>;
  if (nslot <= 0) return;  // no workgroups ran persistent tiles
  const int nk = p.K / BK;
  const TileScan ts = tile_scan<BM>(p);
  int total = 0;
  for (int x = 0; x < kXcds; ++x) {
    const XcdShare sh = xcd_share(ts.total, x, kXcds, nslot, nk, p);
    if (sh.S > 1) total += sh.tail;
  }
  const int64_t items = (int64_t)total * FR::ITEMS;
  for (int64_t gi = (int64_t)blockIdx.x * kFixupThreads + threadIdx.x; gi < items; gi += (int64_t)gridDim.x * kFixupThreads) {
    int i = (int)(gi / FR::ITEMS);
    const int it = (int)(gi % FR::ITEMS);
    int x = 0;
    XcdShare sh = xcd_share(ts.total, 0, kXcds, nslot, nk, p);
    for (;;) {
      const int n = sh.S > 1 ? sh.tail : 0;
      if (i < n || x == kXcds - 1) break;
      i -= n;
      sh = xcd_share(ts.total, ++x, kXcds, nslot, nk, p);
    }
    Tile tl;
    if (!tile_of<BM, BNF>(p, ts, sh.lo + sh.rounds * nslot + i, tl)) continue;
    int piece = 0;
    fixup_item<BM, BNF, NB, ACT, Q8>(p, tl, it, [&](int64_t& slot) {
      if (piece >= sh.S) return false;
      slot = (int64_t)x * nslot + (int64_t)piece * sh.tail + i;
      ++piece;
      return true;
    });
  }
}
template <int BM, int BNF, int NB, int ACT, int BK, bool Q8>
__global__ __launch_bounds__(kFixupThreads) void k_gemm_tail_reduce(const GemmParams p, int nslot) {
  if (fixup_idle(p)) return;
  tail_reduce<BM, BNF, NB, ACT, BK, Q8>(p, nslot);
}

// Stream-K fix-up: for every stream-K tile cut by a range boundary, sums the partials of
// the workgroups that share it in workgroup order and stores the tile. Grid-stride over
// (stream-K tile, fix-up thread), wave-uniform tiles as above.
template <int BM, int BNF, int NB, int ACT, int BK, bool Q8>
__device__ __forceinline__ void streamk_reduce(const GemmParams& p, const int grid) {
  using FR = Frag<BM, BNF, NB, Q8>;
  if (grid <= 0) return;  // no workgroups ran stream-K tiles
  const int nk = p.K / BK;
  const TileScan ts = tile_scan<BM>(p);
  const SkPlan sk = sk_plan(ts.total, grid, nk);
  const int64_t items = (int64_t)(ts.total - sk.dp) * FR::ITEMS;
  for (int64_t gi = (int64_t)blockIdx.x * kFixupThreads + threadIdx.x; gi < items; gi += (int64_t)gridDim.x * kFixupThreads) {
    const int ls = (int)(gi / FR::ITEMS), it = (int)(gi % FR::ITEMS);
    const int64_t wa = sk_owner((int64_t)ls * nk, sk.W, sk.g), wb = sk_owner((int64_t)(ls + 1) * nk - 1, sk.W, sk.g);
    if (wa == wb) continue;  // stored directly by its only workgroup
    Tile tl;
    if (!tile_of<BM, BNF>(p, ts, sk.dp + ls, tl)) continue;
    int64_t w = wa;
    fixup_item<BM, BNF, NB, ACT, Q8>(p, tl, it, [&](int64_t& slot) {
      for (; w <= wb; ++w) {
        const int64_t b0 = sk_begin(w, sk.W, sk.g);
        if (sk_begin(w + 1, sk.W, sk.g) <= b0) continue;  // empty range (fewer items than workgroups)
        slot = 2 * w + ((int64_t)ls == b0 / nk ? 0 : 1);
        ++w;
        return true;
      }
      return false;
    });
  }
}
template <int BM, int BNF, int NB, int ACT, int BK, bool Q8>
__global__ __launch_bounds__(kFixupThreads) void k_gemm_streamk_reduce(const GemmParams p, int grid) {
  if (fixup_idle(p)) return;
  if (p.dual && skinny_wide(p, grid)) return;  // the dual skinny kernel ran whole wide tiles
  streamk_reduce<BM, BNF, NB, ACT, BK, Q8>(p, grid);
}

// ---- mixed tile heights ----------------------------------------------------------------
// A launch whose experts' rows mostly fill 256-row tiles, but where some experts end in a
// small remainder (1..64 rows past their last whole 256-row block, or fewer than 65 rows
// in all): a 256-row tile over such a remainder still streams its whole weight panel
// through LDS for a few rows. The workgroups of each XCD may instead split into two shares
// that run concurrently: the big share runs the 256-row tiles of all other rows (persistent
// XCD schedule, tail split along K), the small share runs 64-row tiles (twice as wide) over
// the small remainders with stream-K. Each share's work is estimated as its tiles x the
// elements one tile copies into LDS per row of a K slice, a small tile's weighted by
// MOE_MIX_SHARED_COST percent when its expert also has 256-row tiles (the same weight
// panels pass through L2 for those) and by MOE_MIX_LONE_COST percent when not (its panels
// come from HBM alone); measured: a small share sized too small leaves it the slower one by
// far, one sized too large costs little. The size of the small share (whole XCD slots, or
// none: then every row runs on 256-row tiles as in k_gemm_bf16) is the one with the earliest
// estimated finish of the slower share. Integer arithmetic on counts[] only, so the GEMM and
// its fix-up agree; every output element is one fp32 sum over K in a fixed order whatever
// the split.
#ifndef MOE_MIX_SHARED_COST
#define MOE_MIX_SHARED_COST 70
#endif
#ifndef MOE_MIX_LONE_COST
#define MOE_MIX_LONE_COST 100
#endif
constexpr int kMixRemMax = 64;

// The tile list of one share: part 0 (every row on 256-row tiles), 1 (big share) or 2
// (small share).
// Tile shapes of a mixed launch (template arguments of the functions below): the big
// share's 256 x (NB x BNF_B) tiles with BK_B-deep slices in STAGES_B stages, the small
// share's 64 x (NB x BNF_S) tiles with BK_S-deep slices in STAGES_S stages; Q8: int8
// weights with column scales.
template <int NB, int BNF_B, int BNF_S>
__device__ __forceinline__ GemmParams mixed_view(const GemmParams& p, int part) {
  GemmParams q = p;
  q.part = part;
  q.rem_max = kMixRemMax;
  q.n_tiles = p.N / (part == 2 ? BNF_S : BNF_B);
  return q;
}

// Estimated finish time of a split with s of the n slots per XCD in the small share, as a
// fraction num / den (the slower share's work per slot).
struct MixTime {
  int64_t num, den;
};
__device__ __forceinline__ bool mix_faster(MixTime a, MixTime b) { return a.num * b.den < b.num * a.den; }
__device__ __forceinline__ MixTime mix_time(int64_t wb, int64_t ws, int s, int n) {
  if (s == 0) return MixTime{wb, n};
  const MixTime big{wb, n - s}, small{ws, s};
  if (s == n) return small;
  return mix_faster(big, small) ? small : big;
}

// Workgroups of the small share (a multiple of kXcds, 0 for none) out of G: the better of
// no split and the two whole slot counts around the balance point
// s* = n ws / (wb + ws), where both shares' work per slot is equal. A tile's work is the
// bytes it copies into LDS per row of a K slice (bf16 activation rows, weights of WB bytes).
template <int NB, int BNF_B, int BNF_S, bool Q8>
__device__ __forceinline__ int mixed_small_wgs(const GemmParams& p, int G) {
  constexpr int WB = Q8 ? 1 : 2;
  // weighted small tiles: one 64-row tile row per expert with a small remainder (lane e =
  // expert e, E <= 64), summed over the wave in a fixed butterfly order
  const int lane = lane_id();
  int c = lane < p.E ? p.counts[lane] : 0;
  c = c < 0 ? 0 : c;
  const int rem = c % kMixBlockRows;
  int64_t wsl = (rem > 0 && rem <= kMixRemMax) ? (c > rem ? MOE_MIX_SHARED_COST : MOE_MIX_LONE_COST) : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsl += __shfl_xor(wsl, off);
  const int n = G / kXcds;
  if (wsl == 0 || n < 2) return 0;
  const int t0 = tile_scan<256>(mixed_view<NB, BNF_B, BNF_S>(p, 0)).total;
  const int tb = tile_scan<256>(mixed_view<NB, BNF_B, BNF_S>(p, 1)).total;
  const int64_t cb = (int64_t)(256 * 2 + NB * BNF_B * WB) * 100;
  const int64_t wb = (int64_t)tb * cb, w0 = (int64_t)t0 * cb;
  const int64_t ws = wsl * (p.N / BNF_S) * (64 * 2 + NB * BNF_S * WB);
  const int smax = tb > 0 ? n - 1 : n;
  int lo = (int)((int64_t)n * ws / (wb + ws));
  lo = lo < 1 ? 1 : (lo > smax ? smax : lo);
  const int hi = lo < smax ? lo + 1 : lo;
  int best = 0;
  MixTime bt = mix_time(w0, 0, 0, n);
  const MixTime tl = mix_time(wb, ws, lo, n), th = mix_time(wb, ws, hi, n);
  if (mix_faster(tl, bt)) { best = lo; bt = tl; }
  if (mix_faster(th, bt)) { best = hi; bt = th; }
  return __builtin_amdgcn_readfirstlane(best * kXcds);  // wave-uniform: the schedule stays scalar
}

// The fp32 partial slots of the small share follow the big share's.
template <int NB, int BNF_B, bool Q8>
__device__ __forceinline__ float* mixed_small_partial(const GemmParams& p, int gb) {
  return p.partial + (size_t)gb * 8 * Frag<256, BNF_B, NB, Q8>::NACC * 64;
}

template <int ACT, int NB, int BNF_B, int BK_B, int STAGES_B, int BNF_S, int BK_S, int STAGES_S, bool Q8, bool GA>
__global__ __launch_bounds__(512, 1) void k_gemm_mixed(const GemmParams p) {
  static_assert(2 * Frag<64, BNF_S, NB, Q8>::NACC <= Frag<256, BNF_B, NB, Q8>::NACC,
                "two small-tile partial slots per big-tile slot");
  constexpr int EL_B = Ring<256, BNF_B, NB, BK_B, STAGES_B, false, Q8>::EL;
  constexpr int EL_S = Ring<64, BNF_S, NB, BK_S, STAGES_S, true, Q8>::EL;
  __shared__ __attribute__((aligned(1024))) bf16 ring[EL_B > EL_S ? EL_B : EL_S];
  const int G = gridDim.x;
  const int gs = mixed_small_wgs<NB, BNF_B, BNF_S, Q8>(p, G);
  const int gb = G - gs;
  const int b = blockIdx.x;  // b % kXcds is the XCD in both shares (gb % kXcds == 0)
  if (b == 0 && threadIdx.x < 64) {  // before the tiles, so none of it stays live across them
    const bool big = gb > 0 && persistent_splits<256, BK_B>(mixed_view<NB, BNF_B, BNF_S>(p, gs > 0 ? 1 : 0), gb);
    set_fixup(p, big || streamk_partials<64, BK_S>(mixed_view<NB, BNF_B, BNF_S>(p, 2), gs));
  }
  if (b < gb) {
    gemm_tiles<256, BNF_B, NB, ACT, BK_B, STAGES_B, false, Q8, GA>(mixed_view<NB, BNF_B, BNF_S>(p, gs > 0 ? 1 : 0),
                                                                   ring, b, gb);
  } else {
    GemmParams q = mixed_view<NB, BNF_B, BNF_S>(p, 2);
    q.partial = mixed_small_partial<NB, BNF_B, Q8>(p, gb);
    gemm_tiles<64, BNF_S, NB, ACT, BK_S, STAGES_S, true, Q8, GA>(q, ring, b - gb, gs);
  }
}

// Fix-up of a mixed launch of G workgroups: the big share's tail pieces, then the small
// share's stream-K partials (disjoint rows and partial slots).
template <int ACT, int NB, int BNF_B, int BK_B, int BNF_S, int BK_S, bool Q8>
__global__ __launch_bounds__(kFixupThreads) void k_gemm_mixed_reduce(const GemmParams p, int G) {
  if (fixup_idle(p)) return;
  const int gs = mixed_small_wgs<NB, BNF_B, BNF_S, Q8>(p, G);
  const int gb = G - gs;
  tail_reduce<256, BNF_B, NB, ACT, BK_B, Q8>(mixed_view<NB, BNF_B, BNF_S>(p, gs > 0 ? 1 : 0), gb / kXcds);
  GemmParams q = mixed_view<NB, BNF_B, BNF_S>(p, 2);
  q.partial = mixed_small_partial<NB, BNF_B, Q8>(p, gb);
  streamk_reduce<64, BNF_S, NB, ACT, BK_S, Q8>(q, gs);
}

// Compute units of the first device asked (a launch size only: every kernel is correct for
// any grid, so a device with another count runs correctly, just less well balanced).
// Atomic: host threads may launch concurrently.
std::atomic<int> g_num_cus{0};

int persistent_grid(int64_t tiles_bound) {
  int cus = g_num_cus.load(std::memory_order_relaxed);
  if (cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus.store(n, std::memory_order_relaxed);
    cus = n;
  }
  int64_t g = tiles_bound < cus ? tiles_bound : cus;
  if (g > (int64_t)kGemmPartialUnits) g = kGemmPartialUnits;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)g;
}

// The fix-up word behind the partial tiles (null without a partial buffer).
GemmParams with_fixup(const GemmParams& p) {
  GemmParams q = p;
  q.fixup = p.partial != nullptr
                ? reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(p.partial) + kGemmPartialBytes)
                : nullptr;
  return q;
}

template <int BM, int BNF, int NB, int ACT, int BK, int STAGES, bool STREAMK, bool Q8>
hipError_t launch_act(const GemmParams& p0, int64_t bound, hipStream_t s) {
  const GemmParams p = with_fixup(p0);
  // fp32 partial tiles: 8 waves x NACC accumulators x 64 lanes per slot; stream-K uses two
  // slots per workgroup, the tail split one.
  using FR = Frag<BM, BNF, NB, Q8>;
  constexpr size_t kSlotBytes = (size_t)8 * FR::NACC * 64 * sizeof(float);
  static_assert((STREAMK ? 2 : 1) * kGemmPartialUnits * kSlotBytes <= kGemmPartialBytes, "partial scratch");
  // Fix-up grid: at most `grid` split tiles (tail tiles < one round; stream-K tiles < G).
  auto fixup_grid = [&](int grid) {
    const int64_t threads = (bound < grid ? bound : grid) * (int64_t)FR::ITEMS;
    const int64_t wg = (threads + kFixupThreads - 1) / kFixupThreads;
    return (unsigned)(wg < 2048 ? wg : 2048);
  };
  if constexpr (STREAMK) {
    // Every compute unit takes an equal share of the K slices.
    const int grid = persistent_grid(1 << 30);
    hipLaunchKernelGGL((k_gemm_bf16<BM, BNF, NB, ACT, BK, STAGES, true, Q8>), dim3(grid), dim3(512), 0, s, p);
    hipLaunchKernelGGL((k_gemm_streamk_reduce<BM, BNF, NB, ACT, BK, Q8>), dim3(fixup_grid(grid)), dim3(kFixupThreads), 0, s, p,
                       grid);
  } else {
    const int grid = persistent_grid(bound);
    bool gathered = false;
    if constexpr (NB == 2) {
      if (p.row_token != nullptr) {
        hipLaunchKernelGGL((k_gemm_bf16<BM, BNF, NB, ACT, BK, STAGES, false, Q8, true>), dim3(grid), dim3(512), 0, s, p);
        gathered = true;
      }
    }
    if (!gathered)
      hipLaunchKernelGGL((k_gemm_bf16<BM, BNF, NB, ACT, BK, STAGES, false, Q8>), dim3(grid), dim3(512), 0, s, p);
    if (p.partial != nullptr)
      hipLaunchKernelGGL((k_gemm_tail_reduce<BM, BNF, NB, ACT, BK, Q8>), dim3(fixup_grid(grid)), dim3(kFixupThreads), 0, s, p,
                         grid / kXcds);
  }
  return hipGetLastError();
}

template <int BM, int BNF, int NB, int BK = MOE_GEMM_BK, int STAGES = MOE_GEMM_STAGES, bool STREAMK = false,
          bool Q8 = false>
hipError_t launch_bf16(const GemmParams& p, int act, int64_t mtiles, hipStream_t s) {
  const int64_t bound = mtiles * p.n_tiles;
  if (bound <= 0) return hipSuccess;
  if constexpr (NB == 2) {
    if (act == ACT_SILU) return launch_act<BM, BNF, 2, ACT_SILU, BK, STAGES, STREAMK, Q8>(p, bound, s);
    if (act == ACT_GELU_ERF) return launch_act<BM, BNF, 2, ACT_GELU_ERF, BK, STAGES, STREAMK, Q8>(p, bound, s);
    return launch_act<BM, BNF, 2, ACT_GELU_TANH, BK, STAGES, STREAMK, Q8>(p, bound, s);
  } else {
    return launch_act<BM, BNF, 1, ACT_SILU, BK, STAGES, STREAMK, Q8>(p, bound, s);
  }
}

// Skinny regime (every expert has at most 64 rows, e.g. decode): 64-row tiles, a deeper
// ring (weights stream from HBM with little compute per slice) and stream-K balancing.
constexpr int kSkinnyRows = 64;
#ifndef MOE_SKINNY_BNF
#define MOE_SKINNY_BNF 128
#endif
#ifndef MOE_SKINNY_BK
#define MOE_SKINNY_BK 64
#endif
#ifndef MOE_SKINNY_STAGES
#define MOE_SKINNY_STAGES 4
#endif
bool skinny(const FfnArgs& a) { return a.partial != nullptr && a.max_rows_per_expert <= kSkinnyRows; }

// The dual-width skinny up-projection and its stream-K fix-up (narrow tiles only).
template <int ACT>
hipError_t launch_dual_act(const GemmParams& p0, int64_t bound, hipStream_t s) {
  const GemmParams p = with_fixup(p0);
  using FR = Frag<64, 128, 2, false>;
  const int grid = persistent_grid(1 << 30);
  const int64_t threads = (bound < grid ? bound : grid) * (int64_t)FR::ITEMS;
  const int64_t wg = (threads + kFixupThreads - 1) / kFixupThreads;
  hipLaunchKernelGGL(k_gemm_skinny_dual<ACT>, dim3(grid), dim3(512), 0, s, p);
  hipLaunchKernelGGL((k_gemm_streamk_reduce<64, 128, 2, ACT, 64, false>), dim3((unsigned)(wg < 2048 ? wg : 2048)),
                     dim3(kFixupThreads), 0, s, p, grid);
  return hipGetLastError();
}
hipError_t launch_skinny_dual(const GemmParams& p, int act, int64_t bound, hipStream_t s) {
  if (bound <= 0) return hipSuccess;
  if (act == ACT_SILU) return launch_dual_act<ACT_SILU>(p, bound, s);
  if (act == ACT_GELU_ERF) return launch_dual_act<ACT_GELU_ERF>(p, bound, s);
  return launch_dual_act<ACT_GELU_TANH>(p, bound, s);
}

// Mixed-height launch and its fix-up (one launch each).
template <int ACT, int NB, int BNF_B, int BK_B, int STAGES_B, int BNF_S, int BK_S, int STAGES_S, bool Q8, bool GA>
hipError_t launch_mixed_act(const GemmParams& p0, int64_t bound, hipStream_t s) {
  const GemmParams p = with_fixup(p0);
  using FR = Frag<256, BNF_B, NB, Q8>;
  const int grid = persistent_grid(1 << 30);
  const int64_t threads = (bound < grid ? bound : grid) * (int64_t)FR::ITEMS;
  const int64_t wg = (threads + kFixupThreads - 1) / kFixupThreads;
  hipLaunchKernelGGL((k_gemm_mixed<ACT, NB, BNF_B, BK_B, STAGES_B, BNF_S, BK_S, STAGES_S, Q8, GA>), dim3(grid),
                     dim3(512), 0, s, p);
  hipLaunchKernelGGL((k_gemm_mixed_reduce<ACT, NB, BNF_B, BK_B, BNF_S, BK_S, Q8>), dim3((unsigned)(wg < 2048 ? wg : 2048)),
                     dim3(kFixupThreads), 0, s, p, grid);
  return hipGetLastError();
}

// Gated up-projection, bf16 weights: 256 x (2 x 128) tiles (the split ring) beside
// 64 x (2 x 256) tiles (32-deep slices).
template <int ACT, bool GA>
hipError_t launch_mixed_up_bf16(const GemmParams& p, int64_t bound, hipStream_t s) {
  return launch_mixed_act<ACT, 2, 128, MOE_GEMM_BK, MOE_GEMM_STAGES, 256, MOE_DUAL_BK, MOE_DUAL_STAGES, false, GA>(
      p, bound, s);
}
// int8 weights: 256 x (2 x 128) tiles (three stages) beside 64 x (2 x 256) tiles, as their
// launches without the small share.
template <int ACT>
hipError_t launch_mixed_up_q8(const GemmParams& p, int64_t bound, hipStream_t s) {
  return launch_mixed_act<ACT, 2, 128, 64, 3, 256, 64, 4, true, false>(p, bound, s);
}
template <bool GA, bool Q8>
hipError_t launch_mixed_up(const GemmParams& p, int act, int64_t bound, hipStream_t s) {
  if constexpr (Q8) {
    if (act == ACT_SILU) return launch_mixed_up_q8<ACT_SILU>(p, bound, s);
    if (act == ACT_GELU_ERF) return launch_mixed_up_q8<ACT_GELU_ERF>(p, bound, s);
    return launch_mixed_up_q8<ACT_GELU_TANH>(p, bound, s);
  } else {
    if (act == ACT_SILU) return launch_mixed_up_bf16<ACT_SILU, GA>(p, bound, s);
    if (act == ACT_GELU_ERF) return launch_mixed_up_bf16<ACT_GELU_ERF, GA>(p, bound, s);
    return launch_mixed_up_bf16<ACT_GELU_TANH, GA>(p, bound, s);
  }
}

}  // namespace

bool expert_up_gathers(const FfnArgs& a, bool bf16_io) { return bf16_io && a.s1 == nullptr && !skinny(a); }

hipError_t launch_expert_up(const FfnArgs& a, bool bf16_io, hipStream_t s) {
  if (a.x_row_token != nullptr && !expert_up_gathers(a, bf16_io)) return hipErrorInvalidValue;
  if (!bf16_io) return launch_gemm_f32(a, true, s);
  if (a.s1 != nullptr) {
    // int8 weights: 128-column tiles; the halved B bytes per slice allow deeper rings.
    GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / 128, a.rows, a.partial,
                 kSplitMax, a.s1, a.s2};
    if (skinny(a)) {
      // 64-row tiles, 256 columns per matrix, waves 1 x 8: each wave widens distinct
      // weight columns, so the int8 -> bf16 conversion is not repeated across waves.
      p.split_max = 1;
      if (a.F % 256 == 0) {
        p.n_tiles = a.F / 256;
        return launch_bf16<kSkinnyRows, 256, 2, 64, 4, true, true>(p, a.act, max_m_tiles(a, kSkinnyRows), s);
      }
      return launch_bf16<kSkinnyRows, 128, 2, 64, 6, true, true>(p, a.act, max_m_tiles(a, kSkinnyRows), s);
    }
    if (a.F % 256 == 0 && a.partial != nullptr) {  // 64-row tiles for small remainders
      const int64_t bound = max_m_tiles(a, 256) * p.n_tiles;
      if (bound <= 0) return hipSuccess;
      return launch_mixed_up<false, true>(p, a.act, bound, s);
    }
    return launch_bf16<256, 128, 2, 64, 3, false, true>(p, a.act, max_m_tiles(a, 256), s);
  }
  if (skinny(a) && a.F % 256 == 0) {
    GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / 128, a.rows, a.partial, 1};
    p.dual = 1;
    return launch_skinny_dual(p, a.act, max_m_tiles(a, kSkinnyRows) * (a.F / 128), s);
  }
  if (skinny(a)) {
    constexpr int BNF = MOE_SKINNY_BNF;
    GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / BNF, a.rows, a.partial, 1};
    if (a.F % BNF == 0)
      return launch_bf16<kSkinnyRows, BNF, 2, MOE_SKINNY_BK, MOE_SKINNY_STAGES, true>(p, a.act,
                                                                                       max_m_tiles(a, kSkinnyRows), s);
    p.n_tiles = a.F / 128;
    return launch_bf16<kSkinnyRows, 128, 2, 64, 4, true>(p, a.act, max_m_tiles(a, kSkinnyRows), s);
  }
  constexpr int BM = 256, BNF = 128;
  GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / BNF, a.rows, a.partial, kSplitMax,
               nullptr, nullptr, a.x_row_token};
  if (a.F % 256 == 0 && a.partial != nullptr) {  // the small share's stream-K keeps partials
    const int64_t bound = max_m_tiles(a, BM) * p.n_tiles;
    if (bound <= 0) return hipSuccess;
    return a.x_row_token != nullptr ? launch_mixed_up<true, false>(p, a.act, bound, s)
                                    : launch_mixed_up<false, false>(p, a.act, bound, s);
  }
  return launch_bf16<BM, BNF, 2>(p, a.act, max_m_tiles(a, BM), s);
}

// Skinny down-projection (stream-K over 64-row tiles, every expert at most 64 rows).
#ifndef MOE_SKINNY_DOWN_STAGES
#define MOE_SKINNY_DOWN_STAGES 4
#endif
namespace {
hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s) {
  const int bnf = a.D % 256 == 0 ? 256 : 128;
  const GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / bnf, a.rows, a.partial,
                     1, a.s3, nullptr};
  const int64_t mt = max_m_tiles(a, kSkinnyRows);
  if (a.s3 != nullptr) {
    if (bnf == 256) return launch_bf16<kSkinnyRows, 256, 1, 64, 6, true, true>(p, a.act, mt, s);
    return launch_bf16<kSkinnyRows, 128, 1, 64, 8, true, true>(p, a.act, mt, s);
  }
  if (bnf == 256) return launch_bf16<kSkinnyRows, 256, 1, 64, MOE_SKINNY_DOWN_STAGES, true>(p, a.act, mt, s);
  return launch_bf16<kSkinnyRows, 128, 1, 64, 4, true>(p, a.act, mt, s);
}
}  // namespace

hipError_t launch_expert_down(const FfnArgs& a, bool bf16_io, hipStream_t s) {
  if (!bf16_io) return launch_gemm_f32(a, false, s);
  if (skinny(a)) return launch_down_skinny(a, s);
  if (a.s3 != nullptr) {
    GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / 128, a.rows, a.partial,
                 kSplitMax, a.s3, nullptr};
    // (no small share: its int8 64 x 256 tiles copy 24 KB per K slice, too little to keep
    // pace; measured 1.6 against 1.15 ms on the int8 prefill)
    return launch_bf16<256, 128, 1, 64, 4, false, true>(p, a.act, max_m_tiles(a, 256), s);
  }
  constexpr int BM = 256;
  if (a.D % 256 == 0) {
    GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / 256, a.rows, a.partial,
                 kSplitMax};
    if (a.partial == nullptr) return launch_bf16<BM, 256, 1>(p, a.act, max_m_tiles(a, BM), s);
    // 256 x 256 tiles beside 64 x 256 tiles (64-deep slices, four stages)
    const int64_t bound = max_m_tiles(a, BM) * p.n_tiles;
    if (bound <= 0) return hipSuccess;
    return launch_mixed_act<ACT_SILU, 1, 256, MOE_GEMM_BK, MOE_GEMM_STAGES, 256, 64, 4, false, false>(p, bound, s);
  }
  GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / 128, a.rows, a.partial,
               kSplitMax};
  return launch_bf16<BM, 128, 1>(p, a.act, max_m_tiles(a, BM), s);
}

}  // namespace moe
