// gemm_common.h: tile scheduling shared by the grouped-GEMM kernels of the expert FFN.
// (Internal header of the HIP library.)
//
// A grouped GEMM computes, for every expert e, C[rows_e, :] = A[rows_e, :] B_e where
// rows_e = [offsets[e], offsets[e] + counts[e]) and B_e is the expert's [K, N] weight
// (N contiguous). Group sizes live on the device (written by the dispatch), so every
// workgroup derives the tile list itself: a wave-wide inclusive scan of the per-expert
// tile counts (one expert per lane, E <= 64) maps a linear tile id to (expert, n-tile,
// m-tile) with a ballot. Tiles are ordered expert-major, then n-tile, then m-tile, so
// consecutive ids share one weight tile and one expert's activations.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

struct GemmParams {
  const void* A;    // [rows, K]
  const void* B0;   // [E, K, N]
  const void* B1;   // [E, K, N] (gated up-projection only)
  void* C;          // [rows, N]
  const int32_t* offsets;
  const int32_t* counts;
  int E, K, N;
  int n_tiles;      // N / BN
  int64_t rows;     // rows of A and C: tiles never touch rows outside [0, rows)
  float* partial;   // split-K partial tiles (null: no split)
  int split_max;    // most K splits of one tile
  const float* S0;  // [E, N] column scales of int8 B0 (weight-only 8-bit experts; else null)
  const float* S1;  // [E, N] column scales of int8 B1
  const int32_t* row_token;  // or null: A row r of the product is row row_token[r] of A
                             // (rows past an expert's count unread)
  int dual;         // skinny up-projection launched as k_gemm_skinny_dual (its fix-up checks)
  // Row filter of a mixed-height launch (0: every expert's rows). An expert's rows split
  // into whole 256-row blocks plus a remainder; a remainder of 1..rem_max rows is "small".
  // part 1: the rows without small remainders; part 2: only the small remainders (an
  // expert's remainder rows start after its whole blocks).
  int part;
  int rem_max;
  // Word the GEMM kernel sets to 1 if its launch left split-K or stream-K partials for the
  // fix-up kernel, else 0 (the fix-up then returns at once); null: always fix up.
  uint32_t* fixup;
};

constexpr int kMixBlockRows = 256;  // row block of the mixed-height filter

struct Tile {
  int e, m0, mcount, n0;
  int64_t row_base;
};

// Per-wave tile table: lane e holds the inclusive prefix of tile counts of experts 0..e
// and the row count of expert e.
struct TileScan {
  int incl;   // inclusive prefix (lanes >= E hold the total)
  int cnt;    // rows of expert `lane` this launch covers (0 for lanes >= E)
  int skip;   // rows of expert `lane` before the first covered row
  int off;    // first buffer row of expert `lane` (offsets[lane])
  int total;  // number of tiles
};

template <int BM>
__device__ __forceinline__ TileScan tile_scan(const GemmParams& p) {
  const int lane = lane_id();
  TileScan s;
  s.cnt = 0;
  s.off = 0;
  if (lane < p.E) {  // both loads in flight together; tile_of needs no load of its own
    s.cnt = p.counts[lane];
    s.off = p.offsets[lane];
  }
  if (s.cnt < 0) s.cnt = 0;
  s.skip = 0;
  if (p.part != 0) {
    const int rem = s.cnt % kMixBlockRows;
    const bool small = rem > 0 && rem <= p.rem_max;
    if (p.part == 1) {
      if (small) s.cnt -= rem;
    } else {
      s.skip = small ? s.cnt - rem : 0;
      s.cnt = small ? rem : 0;
    }
  }
  int incl = ((s.cnt + BM - 1) / BM) * p.n_tiles;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  s.incl = incl;
  s.total = __shfl(incl, 63);
  return s;
}

// Tile L (0 <= L < total) -> expert, rows and columns. Returns false if L is outside the
// tile list or the expert's rows fall outside [0, rows).
template <int BM, int BN>
__device__ __forceinline__ bool tile_of(const GemmParams& p, const TileScan& s, int L, Tile& t) {
  const int e = __popcll(__ballot(s.incl <= L));
  if (L < 0 || e >= p.E) return false;
  const int prefix = e > 0 ? __shfl(s.incl, e - 1) : 0;
  const int cnt = __shfl(s.cnt, e);
  const int mt_e = (cnt + BM - 1) / BM;
  const int rem = L - prefix;
  const int nt = rem / mt_e;
  const int mt = rem - nt * mt_e;
  t.e = e;
  t.m0 = mt * BM;
  t.mcount = min(BM, cnt - t.m0);
  t.n0 = nt * BN;
  t.row_base = (int64_t)__shfl(s.off, e) + __shfl(s.skip, e) + t.m0;
  if (t.row_base < 0 || t.row_base >= p.rows) return false;
  if (t.row_base + t.mcount > p.rows) t.mcount = (int)(p.rows - t.row_base);
  return true;
}

// Persistent schedule of one XCD's share of the tile list. The tiles [lo, hi) are run by
// nslot workgroups in rounds; the last, partial round (tail tiles) is split along K into
// S pieces when that fills more workgroups, and the pieces are summed afterwards in a
// fixed order (deterministic).
struct XcdShare {
  int lo, hi, rounds, tail, S;
};

__device__ __forceinline__ XcdShare xcd_share(int total, int xcd, int xcds, int nslot, int nk, const GemmParams& p) {
  XcdShare s;
  s.lo = (int)((int64_t)total * xcd / xcds);
  s.hi = (int)((int64_t)total * (xcd + 1) / xcds);
  const int n = s.hi - s.lo;
  s.rounds = n / nslot;
  s.tail = n - s.rounds * nslot;
  s.S = 1;
  if (p.partial != nullptr && s.tail > 0) s.S = max(1, min(min(nslot / s.tail, p.split_max), nk));
  return s;
}

// Upper bound on the m-tiles of all experts, from host-known sizes only.
inline int64_t max_m_tiles(const FfnArgs& a, int BM) {
  const int64_t per_e = (a.max_rows_per_expert + BM - 1) / BM;
  const int64_t by_rows = (a.rows + (int64_t)a.E * (BM - 1)) / BM;
  return per_e * a.E < by_rows ? per_e * a.E : by_rows;
}

hipError_t launch_gemm_f32(const FfnArgs& a, bool up, hipStream_t s);

}  // namespace moe
