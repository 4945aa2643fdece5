// gemm.hip: grouped GEMMs of the expert FFN for gfx950.
//
// Method ("第 12 章 MoE：路由、专家与负载" §12.1 gated FFN f_e(x) = [SiLU(x W1_e) * (x W2_e)] W3_e
// with W1, W2 [D,F] and W3 [F,D]; "第 5 章 model.py 精读·中：MoE 路由与专家" §5.3.5 the same form
// with GELU, and §5.3.2 the expert weights stacked on a leading expert axis):
//   up   : h[r,:]      = act(x_perm[r,:] W1_e) * (x_perm[r,:] W2_e)
//   down : y_perm[r,:] = h[r,:] W3_e
// for the rows r of each expert e (rows [offsets[e], offsets[e] + counts[e])).
//
// Design (bf16): one workgroup of 4 waves (2 x 2) computes a BM x BN output tile of one
// expert with v_mfma_f32_32x32x16_bf16, fp32 accumulation. The up projection keeps two
// accumulator sets (W1 and W2 tiles at the same columns) so act(.)*(.) is applied in
// registers before the single bf16 store of h. Operand tiles are double-buffered in LDS.
// A (activations, K contiguous) is read with 16-byte ds_read_b128 from rows padded by 16
// bytes (bank-conflict free). B (weights, stored N contiguous as [K,N]) is kept in its
// natural layout in LDS and fed to the MFMA with the gfx950 transposing read
// ds_read_b64_tr_b16; its rows are padded to 64 bytes modulo 256 so the 4-row groups of
// a transposing read hit distinct banks. The workgroup -> (expert, n-tile, m-tile) map is
// computed on the device from counts[] with a wave prefix scan, so ragged group sizes
// never need a host synchronisation; m-tiles of one (expert, n-tile) are adjacent so
// concurrent workgroups share each weight tile in L2.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short __attribute__((address_space(3))) * lds_i16_ptr;
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;

struct GemmParams {
  const void* A;    // [rows, K]
  const void* B0;   // [E, K, N]
  const void* B1;   // [E, K, N] (gated only)
  void* C;          // [rows, N]
  const int32_t* offsets;
  const int32_t* counts;
  int E, K, N;
  int n_tiles;
  int64_t rows;     // rows of A and C: tiles never touch rows outside [0, rows)
};

struct Tile {
  int e, m0, mcount, n0;
  int64_t row_base;
};

// Maps the linear tile id L to (expert, m-tile, n-tile). Tiles are ordered expert-major,
// then n-tile, then m-tile. Every wave computes the same result; returns false if L is
// past the last tile.
template <int BM, int BN>
__device__ __forceinline__ bool find_tile(const GemmParams& p, int L, Tile& t) {
  const int lane = lane_id();
  const int c = lane < p.E ? p.counts[lane] : 0;
  const int tiles = ((c + BM - 1) / BM) * p.n_tiles;
  int incl = tiles;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  const int e = __popcll(__ballot(incl <= L));
  if (e >= p.E) return false;
  const int prefix = e > 0 ? __shfl(incl, e - 1) : 0;
  const int cnt = __shfl(c, e);
  const int mt_e = (cnt + BM - 1) / BM;
  const int rem = L - prefix;
  const int nt = rem / mt_e;
  const int mt = rem - nt * mt_e;
  t.e = e;
  t.m0 = mt * BM;
  t.mcount = min(BM, cnt - t.m0);
  t.n0 = nt * BN;
  t.row_base = (int64_t)p.offsets[e] + t.m0;
  if (t.row_base < 0 || t.row_base >= p.rows) return false;
  if (t.row_base + t.mcount > p.rows) t.mcount = (int)(p.rows - t.row_base);
  return true;
}

__device__ __forceinline__ bf16x8 tr_read_b16x8(const bf16* q, int row_stride) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(q));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(q + 4 * row_stride));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int BM, int BN, int BK, bool GATED, int ACT>
__global__ __launch_bounds__(256) void k_gemm_bf16(const GemmParams p) {
  constexpr int NB = GATED ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int SA = BK + 8;   // A row stride in elements (16-byte pad)
  constexpr int SB = BN + 32;  // B row stride in elements (64-byte pad)
  constexpr int A_ELEMS = BM * SA, B_ELEMS = BK * SB;
  constexpr int STAGE = A_ELEMS + NB * B_ELEMS;
  constexpr int A_LD = BM * BK / 8 / 256;  // 16-byte chunks per thread
  constexpr int B_LD = BK * BN / 8 / 256;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(BK % 16 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  Tile tl;
  if (!find_tile<BM, BN>(p, blockIdx.x, tl)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int K = p.K, N = p.N;

  const bf16* Ag = reinterpret_cast<const bf16*>(p.A) + tl.row_base * K;
  const int64_t boff = (int64_t)tl.e * K * N + tl.n0;
  const bf16* Bg[NB];
  Bg[0] = reinterpret_cast<const bf16*>(p.B0) + boff;
  if constexpr (GATED) Bg[1] = reinterpret_cast<const bf16*>(p.B1) + boff;

  // Per-thread chunk coordinates (fixed for the whole K loop).
  int a_goff[A_LD], a_soff[A_LD];
#pragma unroll
  for (int q = 0; q < A_LD; ++q) {
    const int i = tid + 256 * q;
    const int r = i / (BK / 8), c8 = i % (BK / 8);
    const int rr = min(r, tl.mcount - 1);  // rows past the expert's count re-read a valid row
    a_goff[q] = rr * K + c8 * 8;
    a_soff[q] = r * SA + c8 * 8;
  }
  int b_goff[B_LD], b_soff[B_LD];
#pragma unroll
  for (int q = 0; q < B_LD; ++q) {
    const int i = tid + 256 * q;
    const int r = i / (BN / 8), c8 = i % (BN / 8);
    b_goff[q] = r * N + c8 * 8;
    b_soff[q] = r * SB + c8 * 8;
  }

  u32x4 ra[A_LD], rb[NB][B_LD];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q) ra[q] = *reinterpret_cast<const u32x4*>(Ag + a_goff[q] + k0);
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int q = 0; q < B_LD; ++q)
        rb[m][q] = *reinterpret_cast<const u32x4*>(Bg[m] + (int64_t)k0 * N + b_goff[q]);
  };
  auto store_lds = [&](int stage) {
    bf16* As = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) *reinterpret_cast<u32x4*>(As + a_soff[q]) = ra[q];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      bf16* Bs = As + A_ELEMS + m * B_ELEMS;
#pragma unroll
      for (int q = 0; q < B_LD; ++q) *reinterpret_cast<u32x4*>(Bs + b_soff[q]) = rb[m][q];
    }
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

  // Fragment addressing. A: lane -> row (lane % 32), k-half (lane / 32).
  // B (transposing read): 16-lane group G -> n half (G & 1) and k-half (G >> 1); inside the
  // group, lane s supplies row (s / 4) and columns 4 * (s % 4) .. +3 of a 4 x 16 block.
  const int a_frag = (wm * WM + (lane & 31)) * SA + 8 * (lane >> 5);
  const int G = lane >> 4, s = lane & 15;
  const int b_frag = (8 * (G >> 1) + (s >> 2)) * SB + wn * WN + 16 * (G & 1) + 4 * (s & 3);

  const int nk = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const bf16* As = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + a_frag + 32 * i * SA + kk * 16);
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const bf16* Bs = As + A_ELEMS + m * B_ELEMS;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const bf16x8 bfr = tr_read_b16x8(Bs + b_frag + kk * 16 * SB + 32 * j, SB);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr, acc[m][i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue. Accumulator element r of lane: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
  bf16* Cg = reinterpret_cast<bf16*>(p.C) + tl.row_base * N + tl.n0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * WN + 32 * j + (lane & 31);
        if (row < tl.mcount) {
          float v;
          if constexpr (GATED) v = activate<ACT>(acc[0][i][j][r]) * acc[1][i][j][r];
          else v = acc[0][i][j][r];
          Cg[(int64_t)row * N + col] = (bf16)v;
        }
      }
}

// fp32 path: plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 outputs per thread).
template <bool GATED, int ACT>
__global__ __launch_bounds__(256) void k_gemm_f32(const GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = GATED ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN];

  Tile tl;
  if (!find_tile<BM, BN>(p, blockIdx.x, tl)) return;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int K = p.K, N = p.N;
  const float* Ag = reinterpret_cast<const float*>(p.A) + tl.row_base * K;
  const int64_t boff = (int64_t)tl.e * K * N + tl.n0;
  const float* Bg[NB];
  Bg[0] = reinterpret_cast<const float*>(p.B0) + boff;
  if constexpr (GATED) Bg[1] = reinterpret_cast<const float*>(p.B1) + boff;

  float acc[NB][4][4];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + 256 * q;
      const int r = i / BK, c = i % BK;
      const int rr = min(r, tl.mcount - 1);
      As[c][r] = Ag[(int64_t)rr * K + k0 + c];
    }
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = tid + 256 * q;
        const int r = i / BN, c = i % BN;
        Bs[m][r][c] = Bg[m][(int64_t)(k0 + r) * N + c];
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[m][j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[m][j], acc[m][i][j]);
    }
    __syncthreads();
  }
  float* Cg = reinterpret_cast<float*>(p.C) + tl.row_base * N + tl.n0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= tl.mcount) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v;
      if constexpr (GATED) v = activate<ACT>(acc[0][i][j]) * acc[1][i][j];
      else v = acc[0][i][j];
      Cg[(int64_t)row * N + tx * 4 + j] = v;
    }
  }
}

// Upper bound on the m-tiles of all experts, from host-known sizes only.
int64_t max_m_tiles(const FfnArgs& a, int BM) {
  const int64_t per_e = (a.max_rows_per_expert + BM - 1) / BM;
  const int64_t by_rows = (a.rows + (int64_t)a.E * (BM - 1)) / BM;
  return per_e * a.E < by_rows ? per_e * a.E : by_rows;
}

template <int BM, int BN, int BK, bool GATED>
hipError_t launch_bf16(const GemmParams& p, int act, int64_t mtiles, hipStream_t s) {
  const dim3 grid((unsigned)(mtiles * p.n_tiles)), block(256);
  if (grid.x == 0) return hipSuccess;
  if constexpr (GATED) {
    if (act == ACT_SILU) hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, true, ACT_SILU>), grid, block, 0, s, p);
    else if (act == ACT_GELU_ERF) hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, true, ACT_GELU_ERF>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, true, ACT_GELU_TANH>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, false, ACT_SILU>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <bool GATED>
hipError_t launch_f32(const GemmParams& p, int act, int64_t mtiles, hipStream_t s) {
  const dim3 grid((unsigned)(mtiles * p.n_tiles)), block(256);
  if (grid.x == 0) return hipSuccess;
  if constexpr (GATED) {
    if (act == ACT_SILU) hipLaunchKernelGGL((k_gemm_f32<true, ACT_SILU>), grid, block, 0, s, p);
    else if (act == ACT_GELU_ERF) hipLaunchKernelGGL((k_gemm_f32<true, ACT_GELU_ERF>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_f32<true, ACT_GELU_TANH>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((k_gemm_f32<false, ACT_SILU>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_up(const FfnArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) {
    constexpr int BM = 128, BN = 128, BK = 64;
    GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / BN, a.rows};
    return launch_bf16<BM, BN, BK, true>(p, a.act, max_m_tiles(a, BM), s);
  }
  constexpr int BM = 64, BN = 64;
  GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / BN, a.rows};
  return launch_f32<true>(p, a.act, max_m_tiles(a, BM), s);
}

hipError_t launch_expert_down(const FfnArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) {
    constexpr int BM = 128, BN = 128, BK = 64;
    GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / BN, a.rows};
    return launch_bf16<BM, BN, BK, false>(p, a.act, max_m_tiles(a, BM), s);
  }
  constexpr int BM = 64, BN = 64;
  GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / BN, a.rows};
  return launch_f32<false>(p, a.act, max_m_tiles(a, BM), s);
}

}  // namespace moe
