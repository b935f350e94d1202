"""Measurement probes, run as ``python -m software_pipelined_tiled_amd.probes <what>``:

    peak    dense MFMA throughput (16x16x32 bf16) in TFLOP/s, 1 and 2 waves per SIMD
    copy    16-byte streaming copy bandwidth in GB/s (read + write)
    lds     the LDS read-pattern kernels, one launch per swizzle (read the counters with rocprofv3)
    fill    global->LDS fill rate per CU: each workgroup re-reading its own 64 KiB (L2-resident),
            and streaming 4 MiB of its own (L2 misses)
"""
from __future__ import annotations

import sys

import torch

from . import _lib


def _timed(fn) -> float:
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    out = fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e), out


def peak(iters: int = 20000) -> dict:
    res = {}
    for w in (1, 2):
        _lib.gemm_probe_mfma_peak(100, w)
        ms, flops = _timed(lambda: _lib.gemm_probe_mfma_peak(iters, w))
        res[f"waves_per_simd_{w}"] = flops / (ms * 1e-3) / 1e12
    return res


def copy(nbytes: int = 1 << 30) -> float:
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    _lib.gemm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes)
    ms, _ = _timed(lambda: _lib.gemm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes))
    return 2 * nbytes / (ms * 1e-3) / 1e9


def fill(iters: int = 2000) -> dict:
    nbytes = 1 << 30
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for name, region in (("l2_resident_64KiB_per_cu", 1 << 16), ("streaming_4MiB_per_cu", 1 << 22)):
        _lib.gemm_probe_fill(src.data_ptr(), nbytes, region, 8)
        ms, moved = _timed(lambda: _lib.gemm_probe_fill(src.data_ptr(), nbytes, region, iters))
        res[name + "_GBps_total"] = moved / (ms * 1e-3) / 1e9
        res[name + "_B_per_ns_per_cu"] = moved / (ms * 1e6) / cus
    return res


def lds(iters: int = 2000) -> None:
    for sw in (-1, 0, 1, 2, 3, 4):
        _lib.gemm_probe_lds_read(sw, iters)
    torch.cuda.synchronize()


if __name__ == "__main__":
    what = sys.argv[1] if len(sys.argv) > 1 else "peak"
    if what == "peak":
        print(peak())
    elif what == "copy":
        print(f"{copy():.1f} GB/s")
    elif what == "fill":
        print(fill())
    elif what == "lds":
        lds()
        print("lds probes launched: swizzles -1, 0, 1, 2, 3, 4 in this order")
    else:
        raise SystemExit(__doc__)
