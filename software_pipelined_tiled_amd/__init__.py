"""Software-pipelined, persistent tiled GEMM C = A·Bᵀ for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libsptgemm.so`` (C ABI in include/gemm.h); this package
is its thin Python face. PyTorch is used only for device memory and streams.
"""
from ._lib import (EXPORTS, GEMM_BF16, GEMM_F16, GEMM_F32, GEMM_LOAD_AUTO, GEMM_LOAD_DMA, GEMM_LOAD_REG,
                   GEMM_LOAD_STAGED, GemmConfig, GemmError, GemmLibraryMissing, gemm_lds_chunk_offset,
                   gemm_plan_create, gemm_plan_describe, gemm_plan_destroy, gemm_plan_parts, gemm_plan_workspace_bytes,
                   gemm_probe_copy, gemm_probe_lds_read, gemm_probe_mfma_peak, gemm_probe_read, gemm_run, gemm_run_noalloc,
                   gemm_pipeline_protocol, gemm_schedule_tile, gemm_select_config, gemm_select_config_status, gemm_select_parts, lib,
                   status_string)
from .torch_api import Plan, matmul

__all__ = ["EXPORTS", "GEMM_BF16", "GEMM_F16", "GEMM_F32", "GEMM_LOAD_AUTO", "GEMM_LOAD_DMA", "GEMM_LOAD_REG",
           "GEMM_LOAD_STAGED", "GemmConfig", "GemmError", "GemmLibraryMissing", "Plan", "gemm_lds_chunk_offset",
           "gemm_plan_create", "gemm_plan_describe", "gemm_plan_destroy", "gemm_plan_parts", "gemm_plan_workspace_bytes",
           "gemm_probe_copy", "gemm_probe_lds_read", "gemm_probe_mfma_peak", "gemm_probe_read", "gemm_run", "gemm_run_noalloc",
           "gemm_pipeline_protocol", "gemm_schedule_tile", "gemm_select_config", "gemm_select_config_status", "gemm_select_parts", "lib", "matmul",
           "status_string"]
