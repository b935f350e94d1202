"""Measurement probes, run as ``python -m software_pipelined_tiled_amd.probes <what>``:

    peak    dense MFMA throughput (16x16x32 bf16) in TFLOP/s, 1 and 2 waves per SIMD
    copy    16-byte streaming copy bandwidth in GB/s (read + write)
    lds     the LDS read-pattern kernels, one launch per swizzle (read the counters with rocprofv3)
    fill    global->LDS fill rate per CU: each workgroup re-reading its own 64 KiB (L2-resident),
            and streaming 4 MiB of its own (L2 misses)
    dma     global->LDS issue rate: 1, 4, 8 or 16 issuing waves per CU, each keeping 1..16 loads in
            flight, L2-resident reads
    ldsbw   LDS read bandwidth per CU: 8 waves per CU, 16 independent ds_read_b128 per wave in flight
    store   epilogue store shapes: rows per store instruction (16, 8, 4, 2) x lane layout, with 1, 8
            or 32 writing workgroups per XCD
    ablation [c3|c4] the stage-count ablation: every tile and ring depth of the menu, persistent (static
            rounds or the dynamic queue) and not, group_m 1 and the 32x32x16 MFMA form, each forced
            through the configuration override;
            one untimed pass, then two alternating passes of 10 launches; prints a markdown table of
            TFLOP/s
    library [c3|c4|c2|c5a|c5b|c5c [launches]] one workload (8192^3 bf16 by default, inputs drawn with
            torch in the workload's distribution) through this library's default plan (for 8192^3
            also its 4-wave 256x256 split-ring plan) and, for context only, torch.mm (the vendor GEMM
            library), in alternating blocks of launches; prints TFLOP/s per block. Run it under
            rocprofv3 --pmc to compare clock, MFMA utilisation and instruction mix per kernel.
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


def dma(iters: int = 1000) -> list[dict]:
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = cus * 65536
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    rows = []
    for waves in (1, 4, 8, 16):
        for depth in (1, 2, 4, 8, 16):
            _lib.gemm_probe_dma_rate(src.data_ptr(), nbytes, waves, depth, 4)
            ms, moved = _timed(lambda: _lib.gemm_probe_dma_rate(src.data_ptr(), nbytes, waves, depth, iters))
            per_cu = moved / (ms * 1e6) / cus
            rows.append({"waves": waves, "depth": depth, "B_per_ns_per_cu": per_cu,
                         "B_per_ns_per_wave": per_cu / waves, "ns_per_load_per_wave": 1024.0 / (per_cu / waves)})
    return rows


def store(iters: int = 20, ldc: int = 32768) -> list[dict]:
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = cus * 256 * ldc
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rows = []
    for r, layout in ((16, 0), (16, 1), (8, 1), (4, 1), (2, 1)):
        for active in (1, 8, 32):
            _lib.gemm_probe_store(dst.data_ptr(), nbytes, ldc, r, layout, active, 2)
            ms, written = _timed(lambda: _lib.gemm_probe_store(dst.data_ptr(), nbytes, ldc, r, layout, active, iters))
            wgs = min(active * 8, cus)
            rows.append({"rows_per_instr": r, "layout": "mfma rows" if layout == 0 else "along a row",
                         "active_per_xcd": active, "us_per_128KiB": ms * 1e3 / iters,
                         "GB_per_s_per_cu": written / wgs / (ms * 1e-3) / 1e9,
                         "GB_per_s_total": written / (ms * 1e-3) / 1e9})
    return rows


def ldsbw(iters: int = 4000) -> dict:
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _lib.gemm_probe_lds_bw(10)
    ms, nbytes = _timed(lambda: _lib.gemm_probe_lds_bw(iters))
    per_cu = nbytes / (ms * 1e6) / cus
    return {"B_per_ns_per_cu": per_cu, "B_per_clk_per_cu_if_2.4GHz": per_cu / 2.4,
            "TB_per_s_total": nbytes / (ms * 1e-3) / 1e12}


LIBRARY_SHAPES = {"c3": (8192, 8192, 8192, torch.bfloat16, "normal"),
                  "c4": (16384, 16384, 1024, torch.bfloat16, "uniform"),
                  "c2": (4096, 4096, 4096, torch.float16, "uniform"),
                  "c5a": (32, 8192, 8192, torch.float16, "uniform"),
                  "c5b": (4093, 5119, 3071, torch.float16, "uniform"),
                  "c5c": (8192, 1024, 28672, torch.float16, "uniform")}


def library(workload: str = "c3", reps: int = 3, launches: int = 6) -> list[dict]:
    from .torch_api import Plan

    M, N, K, dt, dist = LIBRARY_SHAPES[workload]
    g = torch.Generator(device="cuda").manual_seed(0)
    if dist == "normal":
        A = (torch.randn(M, K, device="cuda", generator=g) / K ** 0.5).to(dt)
        B = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(dt)
    else:
        A = (torch.rand(M, K, device="cuda", generator=g) * 2 - 1).to(dt)
        B = (torch.rand(N, K, device="cuda", generator=g) * 2 - 1).to(dt)
    C = torch.empty(M, N, dtype=dt, device="cuda")
    plans = {"default plan": Plan(M, N, K, dt, dt)}
    if workload == "c3":
        four_wave = dict(bm=256, bn=256, bk=64, stages=5, waves=4, mfma=16, persistent=1, group_m=8, load_path=1,
                         grid=0, lds_bytes=0, splits=1)
        plans["4-wave split ring"] = Plan(M, N, K, dt, dt, config=four_wave)
    sp = torch.cuda.current_stream().cuda_stream
    runs = {name: (lambda p=p: p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)) for name, p in plans.items()}
    runs["torch.mm (context)"] = lambda: torch.mm(A, B.t(), out=C)
    rows = []
    for r in range(reps):
        for name, fn in runs.items():
            ms, _ = _timed(lambda: [fn() for _ in range(launches)])
            rows.append({"workload": workload, "rep": r, "kernel": name,
                         "TFLOP/s": 2.0 * M * N * K * launches / (ms * 1e-3) / 1e12})
    for p in plans.values():
        p.close()
    return rows


ABLATION_SHAPES = {"c3": (8192, 8192, 8192, torch.bfloat16, "normal"),
                   "c4": (16384, 16384, 1024, torch.bfloat16, "uniform")}
# (row label, column label, tile, ring depth, waves, K-tile depth, load path, persistent, group_m, MFMA)
ABLATION_ROWS = (
    [("256x256 two-group (8 waves)", c, 256, 256, s, 8, 64, 1, p, g, m) for c, s, p, g, m in
     (("S=2", 2, 1, 8, 16), ("S=5 (split ring)", 5, 1, 8, 16), ("non-persistent, S=5", 5, 0, 8, 16),
      ("group_m = 1, S=5", 5, 1, 1, 16), ("32x32x16 MFMA, S=5", 5, 1, 8, 32))]
    + [("256x256 4-wave", c, 256, 256, s, 4, 64, 1, p, 8, 16) for c, s, p in
       (("S=1 (serial)", 1, 1), ("S=2", 2, 1), ("S=5 (split ring)", 5, 1), ("non-persistent, S=2", 2, 0))]
    + [("256x128", c, 256, 128, s, 4, 64, 1, p, 8, 16) for c, s, p in
       (("S=1 (serial)", 1, 1), ("S=2", 2, 1), ("S=3", 3, 1), ("non-persistent, S=3", 3, 0),
        ("dynamic queue, S=3", 3, 2))]
    + [("128x128", c, 128, 128, s, 4, 64, 1, p, 8, 16) for c, s, p in
       (("S=1 (serial)", 1, 1), ("S=2", 2, 1), ("S=3", 3, 1), ("S=4", 4, 1), ("non-persistent, S=4", 4, 0),
        ("dynamic queue, S=4", 4, 2))]
    + [("128x128 register-staged", "S=2", 128, 128, 2, 4, 64, 2, 1, 8, 16)])


def ablation(workload: str = "c3", passes: int = 2, launches: int = 10) -> str:
    from .torch_api import Plan

    M, N, K, dt, dist = ABLATION_SHAPES[workload]
    g = torch.Generator(device="cuda").manual_seed(0)
    if dist == "normal":
        A = (torch.randn(M, K, device="cuda", generator=g) / K ** 0.5).to(dt)
        B = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(dt)
    else:
        A = (torch.rand(M, K, device="cuda", generator=g) * 2 - 1).to(dt)
        B = (torch.rand(N, K, device="cuda", generator=g) * 2 - 1).to(dt)
    C = torch.empty(M, N, dtype=dt, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    plans = []
    for row, col, bm, bn, s, w, bk, path, pers, gm, mf in ABLATION_ROWS:
        cfg = dict(bm=bm, bn=bn, bk=bk, stages=s, waves=w, mfma=mf, persistent=pers, group_m=gm, load_path=path,
                   grid=0, lds_bytes=0, splits=1)
        plans.append((row, col, Plan(M, N, K, dt, dt, config=cfg)))
    res = {(r, c): [] for r, c, _ in plans}
    for _, _, p in plans:  # one untimed pass: clocks and caches settle before the first timed launch
        for _ in range(launches):
            p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)
    torch.cuda.synchronize()
    for _ in range(passes):
        for r, c, p in plans:
            p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)
            ms, _ = _timed(lambda p=p: [p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)
                                        for _ in range(launches)])
            res[(r, c)].append(2.0 * M * N * K * launches / (ms * 1e-3) / 1e12)
    for _, _, p in plans:
        p.close()
    out = [f"| {workload}: configuration | TFLOP/s (one per pass) |", "|---|---|"]
    for (r, c), v in res.items():
        out.append(f"| {r}, {c} | " + " / ".join(f"{x:.0f}" for x in v) + " |")
    return "\n".join(out)


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
    elif what == "dma":
        for row in dma():
            print(row)
    elif what == "store":
        for row in store():
            print(row)
    elif what == "ldsbw":
        print(ldsbw())
    elif what == "ablation":
        print(ablation(sys.argv[2] if len(sys.argv) > 2 else "c3"), flush=True)
    elif what == "library":
        for row in library(sys.argv[2] if len(sys.argv) > 2 else "c3",
                           launches=int(sys.argv[3]) if len(sys.argv) > 3 else 6):
            print(row, flush=True)
    elif what == "lds":
        lds()
        print("lds probes launched: swizzles -1, 0, 1, 2, 3, 4 in this order")
    else:
        raise SystemExit(__doc__)
