"""Measurement probes, run as ``python -m software_pipelined_tiled_amd.probes <what>``:

    peak     dense MFMA throughput (16x16x32 bf16) in TFLOP/s, 1 and 2 waves per SIMD
    copy     16-byte streaming copy bandwidth in GB/s (read + write)
    read     16-byte read-only stream over 1 GiB (more than the 256 MB MALL), in GB/s: the HBM read
             ceiling of a memory-bound GEMM's operand stream
    lds      the LDS read-pattern kernels, one launch per swizzle (read the counters with rocprofv3)
    ablation [c3|c4] the stage-count ablation: every tile and ring depth of the menu, persistent (static
             rounds or the dynamic queue) and not, group_m 1 and the 32x32x16 MFMA form, each forced
             through the configuration override; one untimed pass, then two alternating passes of 10
             launches; prints a markdown table of TFLOP/s, then the pipeline Gantt model's prediction
             for each tile's ring depths, fed with the measured serial (S = 1) K-tile time and the MFMA
             peak measured in the same process
"""
from __future__ import annotations

import sys

import torch

from . import _lib
from . import gantt


def _timed(fn):
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


def read(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Best of `reps` timed read streams over `nbytes` (after one untimed pass), in GB/s."""
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    _lib.gemm_probe_read(src.data_ptr(), nbytes)
    best = 0.0
    for _ in range(reps):
        ms, _ = _timed(lambda: _lib.gemm_probe_read(src.data_ptr(), nbytes))
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    return best


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
    + [("128x128 register-staged", c, 128, 128, s, 4, 64, 2, 1, 8, 16) for c, s in
       (("S=1 (serial)", 1), ("S=2", 2))])


def _operands(workload: str):
    M, N, K, dt, dist = ABLATION_SHAPES[workload]
    g = torch.Generator(device="cuda").manual_seed(0)
    if dist == "normal":
        A = (torch.randn(M, K, device="cuda", generator=g) / K ** 0.5).to(dt)
        B = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(dt)
    else:
        A = (torch.rand(M, K, device="cuda", generator=g) * 2 - 1).to(dt)
        B = (torch.rand(N, K, device="cuda", generator=g) * 2 - 1).to(dt)
    return M, N, K, dt, A, B


def gantt_table(workload: str, res: dict, peak_tflops: float, cus: int = 256) -> str:
    """The Gantt model beside the measured ring depths of each 4-wave DMA tile: the MMA time of a
    K-tile at the measured MFMA peak, the load time as the serial K-tile time less that, and the
    model's TFLOP/s for every depth measured with a static persistent grid."""
    M, N, K, _, _ = ABLATION_SHAPES[workload]
    flop = 2.0 * M * N * K
    out = [f"| {workload}: tile | K-tiles per tile, rounds | MMA / load per K-tile (us) | depth | measured TFLOP/s "
           "| model TFLOP/s | model idle |", "|---|---|---|---|---|---|---|"]
    for tile, bm, bn in (("256x256 4-wave", 256, 256), ("256x128", 256, 128), ("128x128", 128, 128)):
        serial = res.get((tile, "S=1 (serial)"))
        if not serial:
            continue
        kt = -(-K // 64)
        tiles = -(-M // bm) * -(-N // bn)
        rounds = -(-tiles // min(tiles, cus))
        t1 = flop / (max(serial) * 1e12)                      # fastest serial launch, seconds
        mma = 2.0 * bm * bn * 64 / (peak_tflops * 1e12 / cus)  # one K-tile at the measured MFMA peak
        load = max(t1 / (rounds * kt) - mma, 0.0)
        for col, vals in sorted((c, v) for (r, c), v in res.items() if r == tile):
            if not col.startswith("S="):
                continue
            depth = int(col.split("=")[1].split()[0])
            if depth > 4:
                continue
            t = gantt.predict_rounds(kt, depth, load, mma, rounds)
            idle = gantt.simulate(kt, depth, load, mma, "serial" if depth == 1 else "prefetch")["idle"]
            out.append(f"| {tile} | {kt}, {rounds} | {mma * 1e6:.3f} / {load * 1e6:.3f} | {depth} | "
                       f"{' / '.join(f'{x:.0f}' for x in vals)} | {flop / t / 1e12:.0f} | {idle:.2f} |")
    return "\n".join(out)


def ablation(workload: str = "c3", passes: int = 2, launches: int = 10) -> str:
    from .torch_api import Plan

    M, N, K, dt, A, B = _operands(workload)
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
    pk = max(peak().values())
    out = [f"| {workload}: configuration | TFLOP/s (one per pass) |", "|---|---|"]
    for (r, c), v in res.items():
        out.append(f"| {r}, {c} | " + " / ".join(f"{x:.0f}" for x in v) + " |")
    out += ["", f"MFMA peak probe, same process: {pk:.0f} TFLOP/s (best of one and two waves per SIMD)", "",
            gantt_table(workload, res, pk)]
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
    elif what == "read":
        print(f"{read():.1f} GB/s")
    elif what == "ablation":
        print(ablation(sys.argv[2] if len(sys.argv) > 2 else "c3"), flush=True)
    elif what == "lds":
        lds()
        print("lds probes launched: swizzles -1, 0, 1, 2, 3, 4 in this order")
    else:
        raise SystemExit(__doc__)
