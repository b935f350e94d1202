// Kernel instantiation tables exported by the .hip translation units to the host plan code.
#pragma once

namespace spt {

struct KernelEntry {
  int bm, bn, bk, stages, waves, load_path;  // load_path: 1 = DMA, 2 = REG
  int lds_bytes;
  const void* fn[2][3];  // __global__ void(GemmArgs), by [input f16/bf16][output f16/bf16/f32]
};

const KernelEntry* dma_kernel_table(int* count);
const KernelEntry* reg_kernel_table(int* count);
const KernelEntry* pp_kernel_table(int* count);  // two wave groups (waves = 8), DMA loads

}  // namespace spt
