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
// Both are plain streaming kernels: 16-byte accesses where alignment allows, one pass over the
// data, a grid-stride loop over 8-element chunks (32-bit chunk indices: the host caps the
// workspace so the counts fit).
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

// dst rows of ldd = Kp elements (16-byte aligned) from src rows of ld elements (any 2-byte
// alignment): dst[row, k] = src[row, k] for k < K, 0 for K <= k < Kp. Chunk q < rows_a * cpr is
// chunk q mod cpr of row q / cpr of A; the chunks after them are B's, the same way (cpr = Kp / 8).
__global__ void __launch_bounds__(256) stage_kernel(StageArgs g) {
  const unsigned cpr = (unsigned)g.ldd >> 3;
  const unsigned na = (unsigned)g.rows_a * cpr;
  const unsigned total = na + (unsigned)g.rows_b * cpr;
  for (unsigned q = blockIdx.x * 256u + threadIdx.x; q < total; q += gridDim.x * 256u) {
    const bool is_a = q < na;
    const unsigned qq = is_a ? q : q - na;
    const unsigned row = qq / cpr;
    const int k = (int)(8u * (qq - row * cpr));
    const unsigned short* s = (const unsigned short*)(is_a ? g.A : g.B) + (size_t)row * (is_a ? g.lda : g.ldb) + k;
    unsigned short h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = k + e < g.K ? s[e] : (unsigned short)0;
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (unsigned)h[2 * e] | ((unsigned)h[2 * e + 1] << 16);
    unsigned short* d = (unsigned short*)(is_a ? g.dA : g.dB) + (size_t)row * g.ldd + k;
    *(u32x4*)d = out;
  }
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
