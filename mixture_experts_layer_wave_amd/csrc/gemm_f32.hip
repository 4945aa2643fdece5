// gemm_f32.hip: grouped GEMMs of the expert FFN for fp32 tensors (gfx950).
//
// Method ("第 12 章 MoE：路由、专家与负载" §12.1 gated FFN f_e(x) = [SiLU(x W1_e) * (x W2_e)] W3_e;
// "第 5 章 model.py 精读·中：MoE 路由与专家" §5.3.5 the GELU form):
//   up   : h[r,:]      = act(x_perm[r,:] W1_e) * (x_perm[r,:] W2_e)
//   down : y_perm[r,:] = h[r,:] W3_e
// Design: a plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 outputs per thread, fp32
// accumulation in K order). The fp32 path serves small layers; the bf16 path is the
// MFMA kernel of gemm_bf16.hip.
#include "gemm_common.h"

namespace moe {
namespace {

// fp32 path: plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 outputs per thread).
template <bool GATED, int ACT>
__global__ __launch_bounds__(256) void k_gemm_f32(const GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = GATED ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN];

  const TileScan ts = tile_scan<BM>(p);
  Tile tl;
  if (!tile_of<BM, BN>(p, ts, blockIdx.x, tl)) return;
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

hipError_t launch_gemm_f32(const FfnArgs& a, bool up, hipStream_t s) {
  constexpr int BM = 64, BN = 64;
  if (up) {
    GemmParams p{a.x_perm, a.w1, a.w2, a.h, a.offsets, a.counts, a.E, a.D, a.F, a.F / BN, a.rows};
    return launch_f32<true>(p, a.act, max_m_tiles(a, BM), s);
  }
  GemmParams p{a.h, a.w3, nullptr, a.y_perm, a.offsets, a.counts, a.E, a.F, a.D, a.D / BN, a.rows};
  return launch_f32<false>(p, a.act, max_m_tiles(a, BM), s);
}

}  // namespace moe
