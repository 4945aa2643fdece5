// combine.hip: gate-weighted combine back to token order, for gfx950.
//
// Method ("第 5 章 model.py 精读·中：MoE 路由与专家" §5.3.5 and §5.8, the output is the gate-weighted
// sum of the selected experts' outputs; "第 12 章 MoE：路由、专家与负载" §12.2, the k
// contributions are accumulated, never overwritten; "8.1 MoE 系列" §2.2 case B, a token
// with every slot dropped gets increment 0):
//   y[t,:] = sum over kept slots j (slot order) of gate_eff[t,j] * y_perm[row_of[t,j],:].
//
// Design: each wave takes a contiguous piece of one token's row; each lane moves 16-byte
// vectors of the k expert rows (all loads first) and accumulates in fp32 in slot order,
// then rounds once to the output type. Each output element is produced by exactly one
// lane, so no atomics and bit-reproducible results.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  static constexpr int n = 8;
  typedef bf16x8 type;
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  typedef f32x4 type;
};

// Vector moves per lane per slot: a wave covers 64 * kU consecutive vectors of one token,
// issuing the loads of all k slots before the first multiply-add.
constexpr int kU = 2;

template <typename T>
__global__ __launch_bounds__(256) void k_combine(const CombineArgs a, int nchunk) {
  typedef typename Vec<T>::type V;
  constexpr int NV = Vec<T>::n;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  const int64_t t = gw / nchunk;
  const int c = (int)(gw % nchunk);
  if (t >= a.N) return;
  int row[kMaxK];
  float g[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    row[j] = (j < a.k) ? a.row_of[t * a.k + j] : -1;
    if (row[j] >= a.rows) row[j] = -1;  // never read outside the expert buffers
    g[j] = (j < a.k) ? a.gate_eff[t * a.k + j] : 0.f;
  }
  const V* yp = reinterpret_cast<const V*>(a.y_perm);
  V* yo = reinterpret_cast<V*>(a.y);
  const int nvec = a.D / NV;
  V v[kMaxK][kU];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = (c * kU + u) * 64 + lane;
      if (row[j] >= 0 && i < nvec) v[j][u] = yp[(int64_t)row[j] * nvec + i];
    }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = (c * kU + u) * 64 + lane;
    if (i >= nvec) break;
    float acc[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (row[j] >= 0) {
#pragma unroll
        for (int q = 0; q < NV; ++q) acc[q] = fmaf(g[j], to_f32(v[j][u][q]), acc[q]);
      }
    }
    V o;
#pragma unroll
    for (int q = 0; q < NV; ++q) o[q] = from_f32<T>(acc[q]);
    yo[t * nvec + i] = o;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool bf16_io, hipStream_t s) {
  const int nvec = a.D / (bf16_io ? Vec<bf16>::n : Vec<float>::n);
  const int nchunk = (nvec + 64 * kU - 1) / (64 * kU);
  const dim3 grid((unsigned)((a.N * nchunk + 3) / 4));
  if (bf16_io) hipLaunchKernelGGL(k_combine<bf16>, grid, dim3(256), 0, s, a, nchunk);
  else hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, a, nchunk);
  return hipGetLastError();
}

}  // namespace moe
