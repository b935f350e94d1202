// Measurement aids: a dense-MFMA throughput kernel (to confirm the peak the roofline divides by)
// and a 16-byte streaming copy (HBM bandwidth, and the reference for scaling memory-traffic
// counters). This translation unit is built with accumulators in VGPRs, which keeps the MFMA
// chains in place without register copies.
#include <hip/hip_runtime.h>

#include <cstdint>

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

// Global->LDS fill probe: one workgroup of 4 waves per CU; each wave issues 16 direct 1 KiB
// loads (buffer_load_dwordx4 ... lds) per iteration into its own 16 KiB of LDS, keeping two
// iterations in flight. Workgroup w reads the `region` bytes at w*region (or all read the first
// `region` bytes when `shared`), wrapping inside them.
typedef __attribute__((address_space(3))) void lds_void_t;
__global__ void __launch_bounds__(256) fill_kernel(const char* src, unsigned nbytes, unsigned region, int shared,
                                                   int64_t iters) {
  __shared__ __attribute__((aligned(1024))) char lds[64 * 1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, (int)nbytes, 0x00020000);
  const unsigned base = shared ? 0u : blockIdx.x * region;
  for (int64_t it = 0; it < iters; ++it) {
    const unsigned it_off = (unsigned)(((uint64_t)it * 65536u) % region);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const unsigned off = base + ((it_off + (unsigned)(w * 16 + j) * 1024u) % region) + 16u * lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds + (w * 16 + j) * 1024), 16, off, 0, 0, 0);
    }
    if (it & 1) __builtin_amdgcn_s_waitcnt(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Global->LDS issue-rate probe: one workgroup of 16 waves per CU, of which the first `waves` issue
// direct 1 KiB loads from the CU's own 64 KiB of src (L2-resident), each keeping D loads in flight
// (a wait for vmcnt <= D-1 after every load). iters x 8 loads per issuing wave.
template <int D>
__global__ void __launch_bounds__(1024, 1) dma_rate_kernel(const char* src, unsigned nbytes, int waves, int64_t iters) {
  __shared__ __attribute__((aligned(1024))) char lds[64 * 1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w >= waves) return;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, (int)nbytes, 0x00020000);
  const unsigned base = blockIdx.x * 65536u;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned chunk = (unsigned)(((it * 8 + j) * 16 + w) & 63);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds + ((w * 8 + j) & 63) * 1024), 16,
                                               base + chunk * 1024u + 16u * lane, 0, 0, 0);
      if constexpr (D == 1) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      if constexpr (D == 2) __builtin_amdgcn_s_waitcnt(0x0F71);   // vmcnt(1)
      if constexpr (D == 4) __builtin_amdgcn_s_waitcnt(0x0F73);   // vmcnt(3)
      if constexpr (D == 8) __builtin_amdgcn_s_waitcnt(0x0F77);   // vmcnt(7)
      if constexpr (D == 16) __builtin_amdgcn_s_waitcnt(0x0F7F);  // vmcnt(15)
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Store-pattern probe: one workgroup of 8 waves per CU; workgroup w writes a 256-row x 512-byte
// block at w*256*ldc, iters times, if w/8 < active (so `active` workgroups per XCD write). Every
// store instruction writes R rows x (1024/R) bytes of 16-byte pieces: lane l takes row l mod R,
// piece l / R (layout 0, the order an MFMA hands out rows), or row l / P, piece l mod P with
// P = 64/R pieces per row (layout 1: consecutive lanes along a row).
__global__ void __launch_bounds__(512, 1) store_pattern_kernel(char* dst, int64_t ldc, int R, int layout, int active,
                                                               int64_t iters) {
  if ((int)(blockIdx.x / 8) >= active) return;
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  const int P = 64 / R, S = 1024 / R;  // pieces per row and bytes per row of one instruction
  const int r = layout == 0 ? lane % R : lane / P, pc = layout == 0 ? lane / R : lane % P;
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(dst + (size_t)blockIdx.x * 256 * ldc, (short)0, (int)(256 * ldc), 0x00020000);
  const u32x4 val = {(unsigned)lane, (unsigned)v, 7u, 9u};
  const int segs = 512 / S;  // row segments of one instruction across a 512-byte row
  for (int64_t it = 0; it < iters; ++it) {
    for (int q = 0; q < 16; ++q) {
      const int row = 32 * v + R * (q / segs) + r, col = S * (q % segs) + 16 * pc;
      __builtin_amdgcn_raw_buffer_store_b128(val, rc, (unsigned)(row * ldc + col), 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// LDS read-bandwidth probe: one workgroup of 8 waves per CU; every wave keeps 16 independent
// ds_read_b128 (conflict-free, 16 bytes per lane at consecutive addresses) in flight, then waits.
__global__ void __launch_bounds__(512, 1) lds_bw_kernel(unsigned* sink, int64_t iters) {
  __shared__ __attribute__((aligned(1024))) char smem[128 * 1024];
  for (int i = threadIdx.x; i < 128 * 1024 / 4; i += 512) ((unsigned*)smem)[i] = (unsigned)i;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned base = (unsigned)(uintptr_t)(const lds_void_t*)smem + (unsigned)(w * 1024 + 16 * lane);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t it = 0; it < iters; ++it) {
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v[j]) : "v"(base), "i"(j * 8192 % 57344));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) sink[0] = 1u;  // keeps the reads alive
}

float* g_sink[64] = {};

}  // namespace

extern "C" gemm_status_t gemm_probe_mfma_peak(int64_t iters, int waves_per_simd, void* stream, double* flops) {
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 2 || !flops) return GEMM_ERR_INVALID;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  if (!g_sink[dev] && hipMalloc(&g_sink[dev], sizeof(float)) != hipSuccess) return GEMM_ERR_HIP;
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
  if (!g_sink[dev] && hipMalloc(&g_sink[dev], sizeof(float)) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  hipLaunchKernelGGL(lds_read_kernel, dim3(cu), dim3(256), 0, (hipStream_t)stream, (unsigned*)g_sink[dev], swizzle,
                     iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_fill(const void* src, int64_t bytes, int64_t region, int64_t iters, void* stream,
                                         double* bytes_moved) {
  if (!src || !bytes_moved || iters < 1 || bytes < 65536 || bytes > 0x7FFF0000LL || region < 65536 ||
      region % 65536 != 0 || region > bytes)
    return GEMM_ERR_INVALID;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  const int shared = region * cu > bytes ? 1 : 0;  // otherwise every workgroup has a region of its own
  hipLaunchKernelGGL(fill_kernel, dim3(cu), dim3(256), 0, (hipStream_t)stream, (const char*)src, (unsigned)bytes,
                     (unsigned)region, shared, iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  *bytes_moved = (double)cu * (double)iters * 65536.0;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_dma_rate(const void* src, int64_t bytes, int waves, int depth, int64_t iters,
                                             void* stream, double* bytes_moved) {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  if (!src || !bytes_moved || iters < 1 || waves < 1 || waves > 16 || bytes > 0x7FFF0000LL ||
      bytes < (int64_t)cu * 65536)
    return GEMM_ERR_INVALID;
  const dim3 g((unsigned)cu), b(1024);
  const hipStream_t st = (hipStream_t)stream;
  const unsigned n = (unsigned)bytes;
  switch (depth) {
    case 1: hipLaunchKernelGGL(dma_rate_kernel<1>, g, b, 0, st, (const char*)src, n, waves, iters); break;
    case 2: hipLaunchKernelGGL(dma_rate_kernel<2>, g, b, 0, st, (const char*)src, n, waves, iters); break;
    case 4: hipLaunchKernelGGL(dma_rate_kernel<4>, g, b, 0, st, (const char*)src, n, waves, iters); break;
    case 8: hipLaunchKernelGGL(dma_rate_kernel<8>, g, b, 0, st, (const char*)src, n, waves, iters); break;
    case 16: hipLaunchKernelGGL(dma_rate_kernel<16>, g, b, 0, st, (const char*)src, n, waves, iters); break;
    default: return GEMM_ERR_INVALID;
  }
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  *bytes_moved = (double)cu * (double)waves * (double)iters * 8.0 * 1024.0;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_store(void* dst, int64_t bytes, int64_t ldc, int rows_per_instr, int layout,
                                          int active_per_xcd, int64_t iters, void* stream, double* bytes_written) {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  const bool r_ok = rows_per_instr == 2 || rows_per_instr == 4 || rows_per_instr == 8 || rows_per_instr == 16;
  if (!dst || !bytes_written || !r_ok || (layout != 0 && layout != 1) || iters < 1 || active_per_xcd < 1 ||
      ldc < 512 || ldc % 16 != 0 || 256 * ldc > 0x7FFF0000LL || bytes < (int64_t)cu * 256 * ldc)
    return GEMM_ERR_INVALID;
  hipLaunchKernelGGL(store_pattern_kernel, dim3((unsigned)cu), dim3(512), 0, (hipStream_t)stream, (char*)dst, ldc,
                     rows_per_instr, layout, active_per_xcd, iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  const int wgs = active_per_xcd * 8 < cu ? active_per_xcd * 8 : cu;
  *bytes_written = (double)wgs * (double)iters * 131072.0;
  return GEMM_OK;
}

extern "C" gemm_status_t gemm_probe_lds_bw(int64_t iters, void* stream, double* bytes_read) {
  if (iters < 1 || !bytes_read) return GEMM_ERR_INVALID;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  if (!g_sink[dev] && hipMalloc(&g_sink[dev], sizeof(float)) != hipSuccess) return GEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GEMM_ERR_HIP;
  hipLaunchKernelGGL(lds_bw_kernel, dim3(cu), dim3(512), 0, (hipStream_t)stream, (unsigned*)g_sink[dev], iters);
  if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  *bytes_read = (double)cu * 512.0 * (double)iters * 16.0 * 16.0;
  return GEMM_OK;
}
