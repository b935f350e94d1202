"""The measurement probes of the C ABI: argument checks on the CPU (they return before any device
call), and on the GPU that each probe runs, that the copy probe copies every byte, and that the MFMA
probe reports the flop count of the work it launched."""
import ctypes

import numpy as np
import pytest
import torch

import software_pipelined_tiled_amd as spt

OK, INVALID = spt._lib.GEMM_OK, spt._lib.GEMM_ERR_INVALID


def test_probe_arguments_rejected_before_any_device_call():
    lib = spt.lib()
    f = ctypes.c_double()
    assert lib.gemm_probe_mfma_peak(0, 1, None, ctypes.byref(f)) == INVALID       # no iterations
    assert lib.gemm_probe_mfma_peak(10, 0, None, ctypes.byref(f)) == INVALID      # waves per SIMD 1 or 2
    assert lib.gemm_probe_mfma_peak(10, 3, None, ctypes.byref(f)) == INVALID
    assert lib.gemm_probe_mfma_peak(10, 1, None, None) == INVALID                 # nowhere to report
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert lib.gemm_probe_copy(None, p, 16, None) == INVALID
    assert lib.gemm_probe_copy(p, None, 16, None) == INVALID
    assert lib.gemm_probe_copy(p, p, 15, None) == INVALID                         # 16-byte chunks only
    assert lib.gemm_probe_copy(p, p, -16, None) == INVALID
    assert lib.gemm_probe_copy(p, p, 0, None) == OK                               # nothing to copy, nothing launched
    assert lib.gemm_probe_read(None, 16, None) == INVALID
    assert lib.gemm_probe_read(p, 24, None) == INVALID
    assert lib.gemm_probe_read(p, 0, None) == OK
    for bad in (-2, 5):
        assert lib.gemm_probe_lds_read(bad, 1, None) == INVALID                   # swizzles -1 .. 4
    assert lib.gemm_probe_lds_read(0, 0, None) == INVALID


gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


@pytest.mark.gpu
@gpu
@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 * (1 << 20) + 48, 64 << 20])
def test_copy_probe_copies_every_byte(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    spt._lib.gemm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert not dst[nbytes:].any(), "nothing written past the end"


@pytest.mark.gpu
@gpu
def test_mfma_and_read_and_lds_probes_run():
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    for w in (1, 2):
        flops = spt._lib.gemm_probe_mfma_peak(50, w)
        # cu x w workgroups of four waves, each 16 MFMAs of 16x16x32 per iteration
        assert flops == pytest.approx(cu * w * 4 * 50 * 16 * (2 * 16 * 16 * 32))
    src = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    spt._lib.gemm_probe_read(src.data_ptr(), 1 << 24)
    for sw in (-1, 0, 1, 2, 3, 4):
        spt._lib.gemm_probe_lds_read(sw, 10)
    torch.cuda.synchronize()
