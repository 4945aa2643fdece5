// moe_device.h: device-side helpers shared by the gfx950 kernels of the MoE layer.
// (Internal header of the HIP library; not part of the C ABI.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16 round-to-nearest-even (gfx950 converts in hardware).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-uniform value (lets the compiler keep it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Activations of the W1 branch. SiLU(z) = z * sigmoid(z); GELU(z) = z * Phi(z) with Phi
// from erf; tanh form 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))).
enum { ACT_SILU = 0, ACT_GELU_ERF = 1, ACT_GELU_TANH = 2 };

template <int ACT>
__device__ __forceinline__ float activate(float z) {
  if constexpr (ACT == ACT_SILU) {
    // hardware exponential and reciprocal: a few fp32 ulp, far below the bf16 rounding of h
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
  } else if constexpr (ACT == ACT_GELU_ERF) {
    // erf by the rational approximation 7.1.26 of Abramowitz & Stegun, Handbook of
    // Mathematical Functions (|error| <= 1.5e-7 for x >= 0), extended as an odd function;
    // far below the bf16 rounding of h.
    const float x = fabsf(z * 0.70710678118654752f);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
    float y = fmaf(1.061405429f, t, -1.453152027f);
    y = fmaf(y, t, 1.421413741f);
    y = fmaf(y, t, -0.284496736f);
    y = fmaf(y, t, 0.254829592f);
    y *= t;
    const float e = 1.0f - y * __expf(-x * x);
    return 0.5f * z * (1.0f + copysignf(e, z));
  } else {
    // 1 + tanh(u) = 2 - 2 / (1 + e^(2u)), with the hardware exponential and reciprocal
    const float c = 0.79788456080286536f;  // sqrt(2/pi)
    const float u = c * (z + 0.044715f * z * z * z);
    return z * (1.0f - __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * u)));
  }
}

}  // namespace moe
