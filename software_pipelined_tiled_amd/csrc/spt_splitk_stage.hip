// The two memory-bound kernels around the GEMM mainloop that a plan's workspace serves:
//
//   * split-K reduction: when the K-loop of every output tile is cut into `splits` ranges
//     ("GEMM II — pipelining with TMA", Step 4's sum over K-tiles, done in several independent
//     pieces), each range leaves an fp32 partial plane; the reduction adds the planes in range
//     order and rounds once into the output type, so the result does not depend on which
//     workgroup finished first and the output is rounded exactly once, as without the split.
//   * operand staging: the direct global->LDS loads move 16-byte chunks, so they need rows that
//     start on 16-byte boundaries and a K that is a multiple of 8. For any other A or B the staging
//     copy writes the operand into rows of Kp = K rounded up to a multiple of 8 elements, with the
//     padding columns zero; the mainloop then runs over Kp, where each padding term adds 0.
//
// Both are plain streaming kernels: one pass over the data, a grid-stride loop over 8-element
// chunks (32-bit chunk indices: the host caps the workspace so the counts fit). The reduction
// uses 16-byte accesses where alignment allows; the staging copy reads each 16-byte chunk of a
// 2-byte-aligned row as the dword-aligned 20 bytes around it and writes it with one 16-byte store.
#include "spt_device.h"
#include "spt_kernels.h"

namespace spt {

template <int OUT>
__device__ __forceinline__ void store_out8(const float (&v)[8], char* row, int j, int N, int es, bool vec) {
  char* p = row + (size_t)j * es;
  if (vec && j + 8 <= N) {
    if constexpr (OUT == 2) {
      f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
      *(f32x4*)p = lo;
      *(f32x4*)(p + 16) = hi;
    } else {
      u32x4 q;
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = OUT == 1 ? pack_bf16(v[2 * e], v[2 * e + 1]) : pack_f16(v[2 * e], v[2 * e + 1]);
      *(u32x4*)p = q;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (j + e >= N) break;
    if constexpr (OUT == 2) {
      ((float*)p)[e] = v[e];
    } else {
      const unsigned h = OUT == 1 ? pack_bf16(v[e], 0.f) : pack_f16(v[e], 0.f);
      ((unsigned short*)p)[e] = (unsigned short)(h & 0xFFFFu);
    }
  }
}

// C[i, j] = out(((P_0[i, j] + P_1[i, j]) + P_2[i, j]) + ... + P_{S-1}[i, j]). Chunk q covers row
// q / cpr, columns 8 (q mod cpr) .. +7 (cpr = ceil(N / 8)). Partial planes have ldw = N rounded up
// to 8, so their chunks are 32-byte aligned; C chunks take vector stores when aligned.
template <int OUT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(ReduceArgs r) {
  constexpr int es = OUT == 2 ? 4 : 2;
  const unsigned cpr = (unsigned)(r.N + 7) >> 3;
  const unsigned total = (unsigned)r.M * cpr;
  const bool vec_rows = ((uintptr_t)r.C % 16 == 0) && ((size_t)r.ldc * es) % 16 == 0;
  for (unsigned q = blockIdx.x * 256u + threadIdx.x; q < total; q += gridDim.x * 256u) {
    const unsigned i = q / cpr;
    const int j = (int)(8u * (q - i * cpr));
    const float* w = r.W + (size_t)i * r.ldw + j;
    f32x4 lo = *(const f32x4*)w, hi = *(const f32x4*)(w + 4);
    for (int s = 1; s < r.splits; ++s) {
      w += r.plane;
      lo += *(const f32x4*)w;
      hi += *(const f32x4*)(w + 4);
    }
    const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    store_out8<OUT>(v, (char*)r.C + (size_t)i * r.ldc * es, j, r.N, es, vec_rows);
  }
}

// 16 bytes at byte offset `off` (any 2-byte alignment) of the buffer `r`, whose first `end` bytes
// are the operand: the dword-aligned 20 bytes that hold them, in two loads, then shifted into place a
// dword at a time (v_alignbyte takes the low 32 bits of a 64-bit pair shifted right by 0..3 bytes).
// A load that reaches past `end` can come back as zeros as a whole, so the chunks at the very end of
// the operand are read an element at a time instead; elements past `end` read as zero.
__device__ __forceinline__ u32x4 load16_unaligned(__amdgpu_buffer_rsrc_t r, unsigned off, unsigned end) {
  const unsigned al = off & ~3u, sh = off & 3u;
  u32x4 o;
  if (al + 20u <= end) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, al, 0, 0);
    const unsigned e = __builtin_amdgcn_raw_buffer_load_b32(r, al + 16u, 0, 0);
    o[0] = __builtin_amdgcn_alignbyte(v[1], v[0], sh);
    o[1] = __builtin_amdgcn_alignbyte(v[2], v[1], sh);
    o[2] = __builtin_amdgcn_alignbyte(v[3], v[2], sh);
    o[3] = __builtin_amdgcn_alignbyte(e, v[3], sh);
  } else {
    unsigned h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = off + 2u * e + 2u <= end ? (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, off + 2u * e, 0, 0) : 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = h[2 * e] | (h[2 * e + 1] << 16);
  }
  return o;
}

// One operand: dst rows of ldd = Kp elements (16-byte aligned) from src rows of ld elements (any
// 2-byte alignment of the base and of ld): dst[row, k] = src[row, k] for k < K, 0 for K <= k < Kp.
// Chunk q (8 elements) is chunk q mod cpr of row q / cpr (cpr = Kp / 8); the grid-stride loop starts
// at chunk `first`. A is dealt from the first thread of the grid up and B from the last one down, so
// the two share one launch and, when the grid holds both, no thread copies two chunks.
__device__ __forceinline__ void stage_operand(const void* src, int ld, void* dst, int rows, int K, int ldd,
                                              unsigned first, unsigned stride) {
  const unsigned cpr = (unsigned)ldd >> 3;
  const unsigned total = (unsigned)rows * cpr;
  if (total == 0) return;
  // the buffer starts at the dword holding src[0]; lead = 0 or 2 bytes before it
  const uintptr_t base = (uintptr_t)src;
  const unsigned lead = (unsigned)(base & 3u);
  const unsigned end = lead + ((unsigned)(rows - 1) * (unsigned)ld + (unsigned)K) * 2u;  // < 2^31 (host check)
  const __amdgpu_buffer_rsrc_t r = make_rsrc((const void*)(base - lead), end);
  for (unsigned q = first; q < total; q += stride) {
    const unsigned row = q / cpr;
    const int k = (int)(8u * (q - row * cpr));
    u32x4 out = load16_unaligned(r, lead + 2u * ((unsigned)row * (unsigned)ld + (unsigned)k), end);
    if (k + 8 > K) {  // the K tail of the row: the padding columns are zero, whatever src holds there
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e >= K) out[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    }
    *(u32x4*)((unsigned short*)dst + (size_t)row * ldd + k) = out;
  }
}

__global__ void __launch_bounds__(256) stage_kernel(StageArgs g) {
  const unsigned t = blockIdx.x * 256u + threadIdx.x, stride = gridDim.x * 256u;
  stage_operand(g.A, g.lda, g.dA, g.rows_a, g.K, g.ldd, t, stride);
  stage_operand(g.B, g.ldb, g.dB, g.rows_b, g.K, g.ldd, stride - 1u - t, stride);
}

const void* splitk_reduce_fn(int out_dtype) {
  switch (out_dtype) {
    case 0: return (const void*)&splitk_reduce_kernel<0>;
    case 1: return (const void*)&splitk_reduce_kernel<1>;
    case 2: return (const void*)&splitk_reduce_kernel<2>;
  }
  return nullptr;
}

const void* stage_fn() { return (const void*)&stage_kernel; }

}  // namespace spt
