#!/usr/bin/env python3
"""Benchmark of the pipelined, persistent tiled GEMM C = A·Bᵀ on one MI355X.

Default workload: M = N = K = 8192, bf16 inputs drawn N(0,1)/sqrt(K), fp32 accumulation, bf16
output. One step is one gemm_run over operands already resident in HBM. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--shape-index I]
                    [--config JSON] [--no-cpu-baseline] [--copy-calibration] [--cold] [--graph]

The roofline object names the bound of the workload: "mfma" (TFLOP/s against the dense peak) when
2MNK at the MFMA peak takes longer than the compulsory bytes at 8 TB/s, else "hbm" (compulsory GB/s
against 8 TB/s). A plan that splits K or stages its operands launches more than one kernel per run;
the per-launch time is then that of the whole run (mainloop plus reduction or staging copy).
With --cold, B rotates over enough copies that the 256 MB MALL cannot hold them, so B comes from HBM.
With --graph, the K timed launches are captured once in a HIP graph and replayed, so a step costs no host
launch (this matters only for the smallest problems, whose kernels are shorter than a launch from Python).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of dense fp16/bf16 MFMA peak (8192³ bf16, 1×MI355X)"
# MI355X dense fp16/bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU (AMD quotes 2.5 PFLOP/s)
PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0
DTYPE_NAME = {0: "f16", 1: "bf16", 2: "f32"}


def load_traffic(workload: str, shape_index: int, kernel: str, cold: bool = False) -> float | None:
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{shape_index}{'_cold_b' if cold else ''}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    from software_pipelined_tiled_amd.profsum import kernel_source_hash

    if d.get("kernel_source_sha") != kernel_source_hash() or d.get("kernel") != kernel:
        return None
    return float(d["hbm_bytes_per_launch"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(a_bits, b_bits, K, in_dt, out_dt, c_gpu, seconds: float, full_seconds: float):
    """The oracle (fp64 triple loop) on the host cores, over rows of the workload, timed; every row it
    computes is also compared with the timed GPU result (c_gpu, the last launch's output bits).

    All rows are computed when that is projected to take at most `full_seconds`, else the leading rows
    that fit in about `seconds`. Returns (cpu_baseline object, parity object)."""
    import numpy as np

    from oracle import oracle as orc

    threads = orc.cpu_share()
    M, N = a_bits.shape[0], b_bits.shape[0]
    block = max(threads, ((1 << 24) // max(N, 1)) // threads * threads)  # about 16 M outputs per call
    parity = {"n_checked": 0, "of": M * N, "max_err_over_tol": 0.0, "n_fail": 0, "worst_index": None,
              "rule": "|C - C_ref| <= 2e-3 (|A||B|^T)_ij + 1 ulp of the output type, every checked output"}
    oracle_s = 0.0

    def run(r0: int, r1: int) -> float:
        t0 = time.perf_counter()
        c_ref, _, t = orc.gemm(a_bits[r0:r1], b_bits, K, in_dt, out_dt, threads=threads, want_s=False)
        dt = time.perf_counter() - t0
        rep = orc.compare(np.ascontiguousarray(c_gpu[r0:r1, :N]), c_ref, t, out_dt, rel=2e-3)
        parity["n_checked"] += rep["n"]
        parity["n_fail"] += rep["n_fail"]
        if rep["n"] and rep["max_ratio"] >= parity["max_err_over_tol"]:
            parity["max_err_over_tol"] = rep["max_ratio"]
            parity["worst_index"] = [int(rep["worst_index"][0]) + r0, int(rep["worst_index"][1])]
        return dt

    # a call costs a fixed part (decoding B, starting threads) plus a part per row of A: two short
    # calls fit both, then the sample is sized
    r1 = min(M, threads)
    r2 = min(M, r1 + 2 * threads)
    t1 = run(0, r1)
    t2 = run(r1, r2) if r2 > r1 else t1
    oracle_s += t1 + t2
    per_row = max((t2 - t1) / max(r2 - 2 * r1, 1), 1e-7) if r2 - r1 > r1 else max(t2 / max(r2 - r1, 1), 1e-7)
    fixed = max(t1 - per_row * r1, 0.0)
    rest = M - r2
    full = fixed * (-(-rest // block)) + per_row * rest <= full_seconds
    end = M if full else min(M, r2 + max(0, int((seconds - oracle_s) / per_row)))
    done = r2
    while done < end:
        nxt = min(end, done + block)
        oracle_s += run(done, nxt)
        done = nxt
    parity["ok"] = parity["n_fail"] == 0
    flop = 2.0 * done * N * K
    # one thread on the smallest workload (256^3, fp16 -> fp32)
    import synthetic_inputs as si
    _, _, k1, a1, b1, i1, o1 = si.workload_operands("c1_256_f16_f32")
    t0 = time.perf_counter()
    orc.gemm(a1, b1, k1, i1, o1, threads=1, want_sums=False)
    st = time.perf_counter() - t0
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    base = {"value": flop / oracle_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"rows 0..{done - 1} of A against all {N} rows of B (K={K}){' (all rows)' if done == M else ''}; "
                       f"{flop:.3e} flop in {oracle_s:.2f} s, fp64 triple loop, {threads} threads"),
            "nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "threads_rule": "the CPUs this process may use, at most 16 (one GPU's share of a shared host)",
            "single_thread_c1": {"seconds": st, "GFLOP/s": 2.0 * 256 ** 3 / st / 1e9,
                                 "workload": "c1_256_f16_f32 (256^3, f16 -> f32), 1 thread"}}
    return base, parity


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3_8192_bf16_bf16")
    ap.add_argument("--shape-index", type=int, default=0)
    ap.add_argument("--config", default=None, help="JSON kernel-config override (ablations)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="oracle time for a row sample when the whole workload would take longer than --cpu-full-seconds")
    ap.add_argument("--cpu-full-seconds", type=float, default=45.0,
                    help="compute (and check) every row with the oracle when that is projected to take at most this")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one 1 GiB copy kernel (reference for memory-traffic counters)")
    ap.add_argument("--no-probes", action="store_true", help="skip the MFMA-peak and HBM-copy probes")
    ap.add_argument("--cold", action="store_true", help="rotate B over copies that together exceed the MALL")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed launches in one HIP graph and replay it (no host launch cost per step)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs each GEMM on a single device, so --gpus N with N > 1 "
              "is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import software_pipelined_tiled_amd as spt
    import synthetic_inputs as si
    from software_pipelined_tiled_amd.profsum import kernel_source_hash, run_kernel_label

    torch.cuda.set_device(0)
    M, N, K, a_bits, b_bits, in_dt, out_dt = si.workload_operands(args.workload, args.shape_index)
    tdt = {0: torch.float16, 1: torch.bfloat16, 2: torch.float32}
    A = torch.from_numpy(a_bits.view(np.int16)).cuda().view(tdt[in_dt])
    B = torch.from_numpy(b_bits.view(np.int16)).cuda().view(tdt[in_dt])
    C = torch.empty((M, N), dtype=tdt[out_dt], device="cuda")
    b_copies = [B]
    if args.cold:  # >= 600 MB of B copies: more than the 256 MB MALL and the 8 x 4 MB of L2
        n_copies = max(2, -(-600_000_000 // max(1, B.numel() * 2)))
        b_copies += [B.clone() for _ in range(n_copies - 1)]
    config = json.loads(args.config) if args.config else None
    plan = spt.Plan(M, N, K, tdt[in_dt], tdt[out_dt], config=config)
    desc = plan.describe()
    parts = plan.parts()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    for i in range(args.warmup):
        plan.run_ptrs(A.data_ptr(), b_copies[i % len(b_copies)].data_ptr(), C.data_ptr(), sp)
    torch.cuda.synchronize()

    # the timed region: K launches back to back between two events on the stream they run on. The
    # mean launch time is taken over this region too: an event pair around every launch adds a few
    # microseconds per step, several percent of a short launch
    graph = None
    if args.graph:
        # the same K launches recorded once and replayed as one graph: a step then costs the GPU's time
        # alone, where a launch from the host loop can cost more than a small problem's kernel
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                plan.run_ptrs(A.data_ptr(), b_copies[i % len(b_copies)].data_ptr(), C.data_ptr(), cap)
        graph.replay()  # one untimed replay
    all_start, all_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    all_start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            plan.run_ptrs(A.data_ptr(), b_copies[i % len(b_copies)].data_ptr(), C.data_ptr(), sp)
    all_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = all_start.elapsed_time(all_end) / args.steps
    avg_launch_ms = ms_per_step
    flop = 2.0 * M * N * K
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12
    run_config = {"plan": desc, "parts": parts}
    kernel_name = run_kernel_label(run_config, DTYPE_NAME[in_dt], DTYPE_NAME[out_dt])
    traffic = load_traffic(args.workload, args.shape_index, kernel_name, args.cold)
    compulsory = (M * K + N * K) * 2 + M * N * (4 if out_dt == 2 else 2)
    hbm_bound = compulsory / (PEAK_HBM_GBS * 1e9) > flop / (PEAK_TFLOPS * 1e12)

    extra = {"avg_launch_ms": avg_launch_ms, "wall_s": wall,
             "pct_of_spec_peak": 100.0 * value / PEAK_TFLOPS,
             "compulsory_hbm_GBps": compulsory / (avg_launch_ms * 1e-3) / 1e9,
             "mfma_achieved_TFLOPs": achieved, "cold_b_copies": len(b_copies) if args.cold else 0,
             "workspace_bytes": plan.workspace_bytes(),
             "gemm_runs": args.warmup + args.steps,
             "kernel_source_sha": kernel_source_hash()}

    if not args.no_probes:
        iters = 20000
        pk_s, pk_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spt.gemm_probe_mfma_peak(100, 2, sp)
        pk_s.record(stream)
        flops = spt.gemm_probe_mfma_peak(iters, 2, sp)
        pk_e.record(stream)
        torch.cuda.synchronize()
        extra["mfma_peak_measured_TFLOPs"] = flops / (pk_s.elapsed_time(pk_e) * 1e-3) / 1e12
    if args.copy_calibration or not args.no_probes:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        spt.gemm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, sp)
        cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cs.record(stream)
        spt.gemm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, sp)
        ce.record(stream)
        torch.cuda.synchronize()
        extra["copy_probe_GBps"] = 2 * nbytes / (cs.elapsed_time(ce) * 1e-3) / 1e9
        # read-only stream over the same 1 GiB (four times the MALL): the HBM read ceiling
        spt.gemm_probe_read(src.data_ptr(), nbytes, sp)
        best = 0.0
        for _ in range(3):
            cs.record(stream)
            spt.gemm_probe_read(src.data_ptr(), nbytes, sp)
            ce.record(stream)
            torch.cuda.synchronize()
            best = max(best, nbytes / (cs.elapsed_time(ce) * 1e-3) / 1e9)
        extra["hbm_read_probe_GBps"] = best
        del src, dst

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[in_dt],
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "in_dtype": DTYPE_NAME[in_dt],
                   "out_dtype": DTYPE_NAME[out_dt], "accumulate": "f32",
                   "distribution": si.WORKLOADS[args.workload]["dist"], "kernel": kernel_name, "plan": desc,
                   **({"parts": parts} if parts["dim"] >= 0 else {}),
                   "b_cache": "cold (rotated copies)" if args.cold else "warm",
                   "launch": "hip graph replay" if args.graph else "host loop"},
        "roofline": ({"bound": "hbm", "achieved": compulsory / (avg_launch_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": compulsory / (avg_launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "traffic": traffic} if hbm_bound else
                     {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": achieved / PEAK_TFLOPS, "traffic": traffic}),
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        # the output of the last timed launch, checked against the oracle rows the baseline computes
        c_bits = C.cpu().numpy() if out_dt == 2 else C.cpu().view(torch.int16).numpy().view(np.uint16)
        line["cpu_baseline"], line["parity"] = cpu_baseline(a_bits, b_bits, K, in_dt, out_dt, c_bits,
                                                            args.cpu_seconds, args.cpu_full_seconds)
    plan.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
