// Kernel instantiation tables exported by the .hip translation units to the host plan code.
#pragma once

namespace spt {

struct KernelEntry {
  int bm, bn, bk, stages, waves, load_path;  // load_path: 1 = DMA, 2 = REG
  int lds_bytes;
  int mfma;  // 16: v_mfma_f32_16x16x32, 32: v_mfma_f32_32x32x16
  const void* fn[2][3];  // __global__ void(GemmArgs), by [input f16/bf16][output f16/bf16/f32]
  // the same kernels loading A ([0]) or B ([1]) with the non-temporal hint; null where not built
  const void* fn_stream[2][2][3] = {};
};

const KernelEntry* dma_kernel_table(int* count);
const KernelEntry* reg_kernel_table(int* count);
const KernelEntry* pp_kernel_table(int* count);  // two wave groups (waves = 8), DMA loads

// Split-K reduction: C (M x N, ldc, output type) from `splits` fp32 partial planes at W, W + plane,
// ... (elements), each M rows of ldw elements (ldw a multiple of 8, W 16-byte aligned).
struct ReduceArgs {
  const float* W;
  long long plane;
  int splits;
  int M, N, ldw;
  void* C;
  int ldc;
};
const void* splitk_reduce_fn(int out_dtype);  // __global__ void(ReduceArgs), 256 threads

// Operand staging: rows_a rows of A (lda) and rows_b rows of B (ldb), K elements each, into dA and
// dB with rows of ldd elements (ldd a multiple of 8 and >= K, dA and dB 16-byte aligned), the
// columns from K to ldd zero.
struct StageArgs {
  const void* A;
  const void* B;
  void* dA;
  void* dB;
  int rows_a, rows_b, K, lda, ldb, ldd;
};
const void* stage_fn();  // __global__ void(StageArgs), 256 threads

}  // namespace spt
