// calib_copy.hip: a device copy whose reads are direct-to-LDS copies (global_load_lds_dwordx4,
// the instruction the grouped GEMMs stream their tiles with) and whose writes are 16-byte
// vector stores. Measurement tooling, not part of the layer: the memory-traffic counters of
// a copy of known size give the factor that turns the counters' readings into bytes, for
// the same read path the GEMM kernels use. Built into its own library (libmoe_calib.so).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

// Each wave moves 1 KB per step: 64 lanes x 16 bytes into its own 1 KB of LDS, then back
// out to dst. bytes is a multiple of 4 KB (one step of a 4-wave workgroup).
__global__ __launch_bounds__(256) void k_copy_lds(const char* src, char* dst, size_t bytes) {
  __shared__ __attribute__((aligned(1024))) char buf[4096];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)buf) + 1024u * w;
  for (size_t off = ((size_t)blockIdx.x * 4 + w) * 1024; off < bytes; off += (size_t)gridDim.x * 4096) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\ts_waitcnt vmcnt(0)" ::"v"(src + off + 16 * lane),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
    const uint4 v = *reinterpret_cast<const uint4*>(buf + 1024 * w + 16 * lane);
    *reinterpret_cast<uint4*>(dst + off + 16 * lane) = v;
  }
}

}  // namespace

// Copies `bytes` (a multiple of 4096) from src to dst (device pointers, 16-byte aligned) on
// `stream` (hipStream_t; NULL = the null stream). Returns 0, or -1 on invalid arguments, -4
// on a launch error.
extern "C" __attribute__((visibility("default"))) int moe_calib_copy_lds(const void* src, void* dst, size_t bytes,
                                                                          void* stream) {
  if (!src || !dst || bytes % 4096 != 0 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
  if (bytes == 0) return 0;
  size_t blocks = bytes / 4096;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_copy_lds, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const char*)src,
                     (char*)dst, bytes);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
