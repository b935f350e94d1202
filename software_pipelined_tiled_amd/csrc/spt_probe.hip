// Measurement aids: a dense-MFMA throughput kernel (to confirm the peak the roofline divides by),
// a 16-byte streaming copy (the reference for scaling memory-traffic counters), a read-only
// 16-byte stream (the HBM read bandwidth a memory-bound GEMM's operand stream can reach) and an
// LDS read-pattern kernel (bank conflicts of candidate LDS layouts). This translation unit is built with accumulators in VGPRs, which keeps the MFMA
// chains in place without register copies.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gemm.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define SPT_MFMA(c) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0)

__global__ void __launch_bounds__(256) mfma_peak_kernel(float* sink, int64_t iters) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) % 3);
    b[e] = (__bf16)(float)(e & 1);
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int64_t it = 0; it < iters; ++it) {
    SPT_MFMA(c0); SPT_MFMA(c1); SPT_MFMA(c2); SPT_MFMA(c3); SPT_MFMA(c4); SPT_MFMA(c5); SPT_MFMA(c6); SPT_MFMA(c7);
    SPT_MFMA(c0); SPT_MFMA(c1); SPT_MFMA(c2); SPT_MFMA(c3); SPT_MFMA(c4); SPT_MFMA(c5); SPT_MFMA(c6); SPT_MFMA(c7);
  }
  const f32x4 s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  if (s[0] + s[1] + s[2] + s[3] == -1.0f) sink[0] = 1.0f;  // never true; keeps the chains alive
}

__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// LDS read-pattern probe: every lane issues ds_read_b128 at the MFMA operand-read address
// (row lane%16, 16-byte chunk lane/16 of a 128-byte-row tile) under swizzle `sw`, or at 16*lane
// for sw < 0. Used with SQ_LDS_BANK_CONFLICT to choose the LDS layout.
__device__ __forceinline__ int probe_swizzle(int sw, int r) {
  switch (sw) {
    case 0: return 0;
    case 1: return r & 7;
    case 2: return (r & 7) ^ ((r >> 3) & 1);
    case 3: return (r >> 1) & 7;
    default: return (r & 3) ^ (((r >> 2) & 1) << 2);
  }
}

__global__ void __launch_bounds__(256) lds_read_kernel(unsigned* sink, int sw, int64_t iters) {
  __shared__ __attribute__((aligned(1024))) char smem[32768];
  for (int i = threadIdx.x; i < 32768 / 4; i += 256) ((unsigned*)smem)[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int addr = sw < 0 ? wave * 1024 + 16 * lane : (wave * 16 + r) * 128 + ((c ^ probe_swizzle(sw, r)) & 7) * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= *(volatile u32x4*)(smem + ((addr + j * 8192) & 32767));
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) sink[0] = 1u;  // keeps the reads alive
}

// HBM read-stream probe: every thread reads 16-byte chunks in a grid-stride loop, eight loads in
// flight per thread, and folds them into one value that is written only if it matches a constant
// no input produces (so the loads cannot be removed). Over a buffer larger than the 256 MB MALL
// this measures the read bandwidth the operand stream of a memory-bound GEMM can reach.
__global__ void __launch_bounds__(256) read16_kernel(const u32x4* __restrict__ src, int64_t n, unsigned* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < n; i += stride) acc ^= src[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) sink[0] = 1u;
}

// One 4-byte sink per device, allocated on the first probe call there; the lock keeps two threads'
// first calls from both allocating it.
float* g_sink[64] = {};
std::mutex g_sink_mu;

bool sink_ready(int dev) {
  std::lock_guard<std::mutex> lock(g_sink_mu);
  return g_sink[dev] || hipMalloc(&g_sink[dev], sizeof(float)) == hipSuccess;
}

}  // namespace

extern "C" gemm_status_t gemm_probe_mfma_peak(int64_t iters, int waves_per_simd, void* stream, double* flops) {
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 2 || !flops) return GEMM_ERR_INVALID;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  if (!sink_ready(dev)) return GEMM_ERR_HIP;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  const int grid = cu * waves_per_simd;  // 4 waves per workgroup: one per SIMD
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, g_sink[dev], iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  *flops = (double)grid * 4.0 * (double)iters * 16.0 * (2.0 * 16 * 16 * 32);
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || bytes % 16 != 0) return GEMM_ERR_INVALID;
  if (bytes == 0) return GEMM_OK;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  const int64_t n = bytes / 16;
  int64_t grid = (n + 255) / 256;
  if (grid > (int64_t)cu * 16) grid = (int64_t)cu * 16;
  hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     (u32x4*)dst, n);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_lds_read(int swizzle, int64_t iters, void* stream) {
  if (swizzle < -1 || swizzle > 4 || iters < 1) return GEMM_ERR_INVALID;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  if (!sink_ready(dev)) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  hipLaunchKernelGGL(lds_read_kernel, dim3(cu), dim3(256), 0, (hipStream_t)stream, (unsigned*)g_sink[dev], swizzle,
                     iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_read(const void* src, int64_t bytes, void* stream) {
  if (!src || bytes < 0 || bytes % 16 != 0) return GEMM_ERR_INVALID;
  if (bytes == 0) return GEMM_OK;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  if (!sink_ready(dev)) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  const int64_t n = bytes / 16;
  int64_t grid = (n + 255) / 256;
  if (grid > (int64_t)cu * 8) grid = (int64_t)cu * 8;
  hipLaunchKernelGGL(read16_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n,
                     (unsigned*)g_sink[dev]);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}
