"""Summaries of rocprofv3 CSV output for the GEMM kernels, as short text files.

    python -m software_pipelined_tiled_amd.profsum kernel-stats STATS_CSV BENCH_JSON OUT_MD --command CMD
        per-kernel durations (rocprofv3 --kernel-trace --stats --output-format csv) next to the
        launch time the benchmark measured with HIP events in the same run

    python -m software_pipelined_tiled_amd.profsum traffic FETCH_CSV WRITE_CSV BENCH_JSON OUT_JSON --command CMD
        HBM bytes per GEMM launch from two counter runs (--pmc FETCH_SIZE, then --pmc WRITE_SIZE) of
        `bench.py --copy-calibration`. Each counter is scaled by what it reads for the 1 GiB copy
        kernel launched in the same run (which moves exactly 2^30 bytes each way).

    python -m software_pipelined_tiled_amd.profsum clock COUNTER_CSV AGENT_CSV BENCH_JSON OUT_MD --command CMD
        average shader clock of each GEMM launch (SQ_BUSY_CYCLES, summed over the shader engines,
        over the launch's duration) and the MFMA utilisation at that clock; the flop count comes
        from SQ_INSTS_VALU_MFMA_MOPS_BF16 or _F16 (512 flop each) and is checked against 2MNK

    python -m software_pipelined_tiled_amd.profsum issue OUT_MD LABEL=CSV[,CSV...] ... --ktiles N --command CMD
        where a mainloop wave's time goes, per wave and K-tile (SQ_WAVE_CYCLES split into issue, waits at
        issue and waits on counters and barriers, with the instruction mix), one column per kernel

    python -m software_pipelined_tiled_amd.profsum lds COUNTER_CSV OUT_MD --command CMD
        bank-conflict ratio SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE of each LDS read-pattern probe
        launched by `python3 -m software_pipelined_tiled_amd.probes lds` (swizzles -1, 0 .. 4 in order)

BENCH_JSON is a file whose last line is the JSON line bench.py printed in that run.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def _code_tokens(text: str) -> str:
    """Source text without comments and whitespace runs: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# the measurement probes are built into the same library but share no code with the GEMM path
_NOT_GEMM = ("spt_probe.hip",)


def kernel_source_hash() -> str:
    """Hash of the GEMM path's sources (comments and layout ignored); a traffic figure is only
    valid for the code it was taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if os.path.basename(p) in _NOT_GEMM:
            continue
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(_code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_prefix(plan: dict) -> str:
    """Start of the demangled template name of the mainloop kernel a plan launches."""
    if plan["load_path"] != 2 and plan["waves"] == 8:
        return f"gemm_pp_kernel<{plan['stages']}, {plan.get('mfma', 16)}, "
    kind = "reg" if plan["load_path"] == 2 else "dma"
    return f"gemm_{kind}_kernel<{plan['bm']}, {plan['bn']}, {plan['bk']}, "


def kernel_matches(plan: dict, name: str) -> bool:
    """Whether a profiler kernel name (demangled, or left mangled as rocprofv3 does for some
    _Float16 instantiations) is the plan's mainloop kernel."""
    pre = kernel_prefix(plan)
    if pre in name:
        return True
    base, args = pre.split("<")
    mangled = base + "I" + "".join(f"Li{a.strip()}E" for a in args.split(",") if a.strip())
    return mangled in name


def plan_parts(config: dict) -> list[dict]:
    """The configurations whose mainloop kernels one gemm_run launches: the plan's, or both parts'
    of a plan cut in two (bench.py records the cut under config["parts"])."""
    parts = config.get("parts")
    if parts and parts.get("dim", -1) >= 0:
        return [parts["first"], parts["second"]]
    return [config["plan"]]


def run_kernel_label(config: dict, in_dt: str, out_dt: str) -> str:
    return " + ".join(kernel_label(p, in_dt, out_dt) for p in plan_parts(config))


def kernel_label(plan: dict, in_dt: str, out_dt: str) -> str:
    """Short name of the mainloop kernel a plan launches, with its configuration (a split-K plan's
    mainloop writes fp32 partial planes)."""
    kind = "reg" if plan["load_path"] == 2 else ("pp" if plan["waves"] == 8 else "dma")
    splits = plan.get("splits", 1)
    out = "f32" if splits > 1 else out_dt
    extra = f",splits={splits}" if splits > 1 else ""
    extra += ",staged" if plan["load_path"] == 3 else ""
    extra += ",mfma32x32x16" if plan.get("mfma", 16) == 32 else ""
    extra += {1: ",stream=A", 2: ",stream=B"}.get(plan.get("stream", 0), "")
    return (f"gemm_{kind}_kernel<{plan['bm']},{plan['bn']},{plan['bk']},{plan['stages']},"
            f"waves={plan['waves']},{in_dt},{out}{extra}>")


def _bench_line(path: str) -> dict:
    with open(path) as f:
        lines = [l for l in f.read().splitlines() if l.strip().startswith("{")]
    if not lines:
        raise SystemExit(f"no JSON line in {path}")
    return json.loads(lines[-1])


def gemm_runs(line: dict) -> int:
    """gemm_run calls in a bench.py process (warm-up and timed steps)."""
    return int(line["extra"].get("gemm_runs", line["steps"] + line["warmup"]))


def _rows(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(stats_csv: str, bench_json: str, out_md: str, command: str) -> None:
    line = _bench_line(bench_json)
    plan = line["config"]["plan"]
    rows = _rows(stats_csv)
    out = [f"# Kernel durations: {line['config']['workload']} ({line['config']['M']}x{line['config']['N']}x"
           f"{line['config']['K']}, {line['config']['in_dtype']} -> {line['config']['out_dtype']})", "",
           f"Command: `{command}`", "",
           f"Plan: {json.dumps(plan)}", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
           "|---|---|---|---|---|---|"]
    plans = plan_parts(line["config"])
    runs = gemm_runs(line)
    gemm_avg = None
    terms = []  # (label, average us, dispatches per run) of the kernels of one gemm_run
    for r in rows:
        name = r.get("Name", r.get("KernelName", "?"))
        avg = float(r["AverageNs"]) / 1e3
        out.append(f"| `{name[:110]}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
        if _run_kernel(plans, name):
            per = max(1, round(int(r["Calls"]) / runs))
            label = next((k for k in AUX_KERNELS if k in name), "mainloop")
            terms.append((label, avg, per))
            if label == "mainloop":
                gemm_avg = avg
    ev_us = line["extra"]["avg_launch_ms"] * 1e3
    run_avg = sum(avg * per for _, avg, per in terms)
    parts = " + ".join(f"{lab} {avg:.1f}" + (f" x {per}" if per > 1 else "") for lab, avg, per in terms)
    ro = line["roofline"]
    out += ["", f"gemm_run time from HIP events in the same run: {ev_us:.1f} us (rocprofv3 average "
                f"{parts} = {run_avg:.1f} us, ratio {ev_us / run_avg:.3f})." if gemm_avg else
            f"gemm_run time from HIP events: {ev_us:.1f} us (kernel not found in the stats).",
            f"Throughput reported by bench.py in this run: {line['value']:.1f} TFLOP/s "
            f"(roofline bound {ro['bound']}: achieved {ro['achieved']:.1f} {ro['unit']}, frac {ro['frac']:.3f})."]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


AUX_KERNELS = ("splitk_reduce_kernel", "stage_kernel")  # the other kernels of one gemm_run


def _run_kernel(plans: list[dict], name: str) -> bool:
    return any(kernel_matches(p, name) for p in plans) or any(k in name for k in AUX_KERNELS)


def _counter_means(path: str, counter: str, plans: list[dict], per_run: int) -> tuple[float, float, int]:
    """Mean value (bytes) of `counter` per gemm_run, summed over the `per_run` dispatches of one
    run (mainloops, reduction, staging copy), skipping the first, cold run; and the copy kernel's."""
    gemm, copy = [], []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"]) * 1024.0  # rocprofv3 reports these two counters in KiB
        if _run_kernel(plans, r["Kernel_Name"]):
            gemm.append(v)
        elif "copy16_kernel" in r["Kernel_Name"]:
            copy.append(v)
    runs = len(gemm) // per_run
    if runs < 2 or not copy:
        raise SystemExit(f"{path}: need >= 2 runs of {per_run} GEMM dispatches and >= 1 copy dispatch with {counter}")
    rest = gemm[per_run:runs * per_run]
    return sum(rest) / (runs - 1), statistics.mean(copy), runs - 1


def _dispatches_per_run(csv_path: str, plans: list[dict], runs: int) -> int:
    """Dispatches of one gemm_run, from the kernel trace or counter file of `runs` runs."""
    n = 0
    for r in _rows(csv_path):
        name = r.get("Kernel_Name", r.get("Name", ""))
        if "Counter_Name" in r and r["Counter_Name"] not in ("FETCH_SIZE", "WRITE_SIZE"):
            continue
        if _run_kernel(plans, name):
            n += 1
    return max(1, round(n / max(runs, 1)))


def traffic(fetch_csv: str, write_csv: str, bench_json: str, out_json: str, command: str) -> None:
    line = _bench_line(bench_json)
    plans = plan_parts(line["config"])
    runs = gemm_runs(line)
    per_run = _dispatches_per_run(fetch_csv, plans, runs)
    f_gemm, f_copy, nf = _counter_means(fetch_csv, "FETCH_SIZE", plans, per_run)
    w_gemm, w_copy, nw = _counter_means(write_csv, "WRITE_SIZE", plans, per_run)
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    c = line["config"]
    out_bytes = 4 if c["out_dtype"] == "f32" else 2
    compulsory = (c["M"] * c["K"] + c["N"] * c["K"]) * 2 + c["M"] * c["N"] * out_bytes
    read, write = f_gemm * f_scale, w_gemm * w_scale
    d = {"workload": c["workload"], "kernel": c["kernel"], "kernel_source_sha": kernel_source_hash(),
         "hbm_bytes_per_launch": read + write, "read_bytes_per_launch": read, "write_bytes_per_launch": write,
         "compulsory_bytes": compulsory, "traffic_over_compulsory": (read + write) / compulsory,
         "fetch_scale": f_scale, "write_scale": w_scale, "gemm_dispatches_averaged": [nf, nw],
         "raw_fetch_size_kib_per_launch": f_gemm / 1024, "raw_write_size_kib_per_launch": w_gemm / 1024,
         "raw_copy_fetch_kib": f_copy / 1024, "raw_copy_write_kib": w_copy / 1024, "command": command}
    with open(out_json, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d, indent=1))


def clock(counter_csv: str, agent_csv: str, bench_json: str, out_md: str, command: str) -> None:
    line = _bench_line(bench_json)
    c = line["config"]
    gpu = next(r for r in _rows(agent_csv) if r.get("Agent_Type") == "GPU")
    n_se, n_cu = int(gpu["Num_Shader_Banks"]), int(gpu["Cu_Count"])
    fmax = float(gpu["Max_Engine_Clk_Fcompute"]) * 1e6
    per = {}
    for r in _rows(counter_csv):
        if not kernel_matches(c["plan"], r["Kernel_Name"]):
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    flop_exact = 2.0 * c["M"] * c["N"] * c["K"]
    out = [f"# Shader clock and MFMA utilisation: {c['workload']} ({c['M']}x{c['N']}x{c['K']}, "
           f"{c['in_dtype']} -> {c['out_dtype']})", "",
           f"Command: `{command}`", "",
           f"Kernel: `{c['kernel']}`; {n_cu} CUs, {n_se} shader engines, peak engine clock {fmax / 1e9:.2f} GHz.",
           "clock = SQ_BUSY_CYCLES / shader engines / duration; MFMA utilisation = achieved flop rate / "
           "(CUs x 4096 flop/clk x clock).", "",
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x CUs x clock x duration), the counter's own measure of",
           "the same thing (empty where the pass did not collect it).", "",
           "| dispatch | duration (us) | TFLOP/s | clock (GHz) | MFMA util. at that clock | MFMA busy | at peak clock | "
           "MFMA flop / 2MNK |",
           "|---|---|---|---|---|---|---|---|"]
    rows = []
    for i, (did, d) in enumerate(sorted(per.items())):
        mops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        tf = flop_exact / d["dur"] / 1e12
        clk = d["SQ_BUSY_CYCLES"] / n_se / d["dur"]
        util = flop_exact / d["dur"] / (n_cu * 4096 * clk)
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES")
        busy_s = f"{busy / (4 * n_cu * clk * d['dur']):.3f}" if busy is not None else ""
        rows.append((tf, clk, util))
        out.append(f"| {did}{' (first)' if i == 0 else ''} | {d['dur'] * 1e6:.1f} | {tf:.1f} | {clk / 1e9:.3f} | "
                   f"{util:.3f} | {busy_s} | {tf * 1e12 / (n_cu * 4096 * fmax):.3f} | {mops * 512 / flop_exact:.3f} |")
    if len(rows) > 1:
        rest = rows[1:]
        out += ["", f"Mean over the launches after the first: {statistics.mean(r[0] for r in rest):.1f} TFLOP/s at "
                    f"{statistics.mean(r[1] for r in rest) / 1e9:.3f} GHz, MFMA utilisation "
                    f"{statistics.mean(r[2] for r in rest):.3f} at that clock."]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


LDS_PATTERNS = {-1: "linear 16*lane (reference)", 0: "none (f = 0)", 1: "row % 8 (the pages' 128-byte swizzle)",
                2: "(row % 8) XOR bit3(row)", 3: "(row / 2) % 8", 4: "(row % 4) XOR (bit2(row) << 2)"}


def lds(counter_csv: str, out_md: str, command: str) -> None:
    per = {}
    for r in _rows(counter_csv):
        if "lds_read_kernel" not in r["Kernel_Name"]:
            continue
        per.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    order = sorted(per)
    if len(order) != len(LDS_PATTERNS):
        raise SystemExit(f"expected {len(LDS_PATTERNS)} probe dispatches, found {len(order)}")
    out = ["# LDS bank conflicts of the MFMA operand read pattern on gfx950", "",
           "Pattern: one ds_read_b128 per lane; lane l reads row l%16 of a tile with 128-byte rows, at logical",
           "16-byte chunk l/16, stored at physical chunk = chunk XOR f(row). One workgroup of 4 waves per CU.",
           "Ratio = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (0 = conflict-free, 0.5 = 2-way, 0.75 = 4-way).", "",
           f"Command: `{command}`", "",
           "| f(row) | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE | ratio |", "|---|---|---|---|"]
    for sw, d in zip(LDS_PATTERNS, order):
        c, a = per[d].get("SQ_LDS_BANK_CONFLICT", 0.0), per[d].get("SQ_LDS_IDX_ACTIVE", 0.0)
        out.append(f"| {LDS_PATTERNS[sw]} | {c:.4g} | {a:.4g} | {c / a if a else float('nan'):.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


# SQ counters that count quad-cycles (4 shader clocks) per wave; multiplied by 4 in the issue summary
QUAD_CYCLE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
                       "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                       "SQ_ACTIVE_INST_MISC", "SQ_INST_CYCLES_VMEM_RD")


def _gemm_counter_means(path: str) -> dict:
    """Per-dispatch means of every counter of the GEMM mainloop kernels in one pass (the first dispatch,
    which warms caches and clocks, left out)."""
    disp = {}
    for r in _rows(path):
        if "gemm_" not in r["Kernel_Name"]:
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(disp)[1:] or sorted(disp)
    names = set().union(*(disp[i] for i in ids)) if ids else set()
    return {c: statistics.mean(disp[i].get(c, 0.0) for i in ids) for c in names}


def issue(runs: list[str], out_md: str, command: str, ktiles: int) -> None:
    """Where a mainloop wave's time goes, per wave and K-tile: one or more counter passes per kernel
    (label=csv[,csv...]); every pass must come from the same workload, whose workgroups each run
    `ktiles` K-tiles. Quad-cycle counters are converted to shader clocks."""
    table = {}
    for spec in runs:
        label, paths = spec.split("=", 1)
        merged = {}
        for path in paths.split(","):
            merged.update(_gemm_counter_means(path))
        table[label] = merged
    counters = sorted(set().union(*table.values()) - {"SQ_WAVES", "SQ_BUSY_CYCLES"})  # not per-wave counts
    out = ["# Per wave and K-tile: issue, stalls and instruction mix of the GEMM mainloop kernels", "",
           f"Command: `{command}`", "",
           f"Means over the dispatches after the first of each pass; per wave and K-tile = counter / SQ_WAVES / "
           f"{ktiles} K-tiles per workgroup. Counters that count quad-cycles (SQ_WAVE_CYCLES, SQ_WAIT_*, "
           "SQ_ACTIVE_INST_*, SQ_INST_CYCLES_VMEM_RD) are multiplied by 4 to give shader clocks; the instruction "
           "counts (SQ_INSTS_*) and SQ_VALU_MFMA_BUSY_CYCLES (clocks, per SIMD) are as counted.", "",
           "| counter | " + " | ".join(table) + " |", "|---|" + "---|" * len(table)]
    for c in counters:
        cells = []
        for label, m in table.items():
            waves = m.get("SQ_WAVES", 0.0)
            if c not in m or waves <= 0:
                cells.append("")
                continue
            v = m[c] / waves / ktiles * (4 if c in QUAD_CYCLE_COUNTERS else 1)
            cells.append(f"{v:.1f}")
        out.append(f"| {c} | " + " | ".join(cells) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernel-stats")
    k.add_argument("stats_csv"), k.add_argument("bench_json"), k.add_argument("out_md")
    k.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv"), t.add_argument("write_csv"), t.add_argument("bench_json"), t.add_argument("out_json")
    t.add_argument("--command", required=True)
    ck = sub.add_parser("clock")
    ck.add_argument("counter_csv"), ck.add_argument("agent_csv"), ck.add_argument("bench_json"), ck.add_argument("out_md")
    ck.add_argument("--command", required=True)
    d = sub.add_parser("lds")
    d.add_argument("counter_csv"), d.add_argument("out_md")
    d.add_argument("--command", required=True)
    iss = sub.add_parser("issue")
    iss.add_argument("out_md"), iss.add_argument("runs", nargs="+", help="label=csv[,csv...] per kernel")
    iss.add_argument("--ktiles", type=int, required=True, help="K-tiles each workgroup runs")
    iss.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.what == "issue":
        issue(a.runs, a.out_md, a.command, a.ktiles)
    elif a.what == "lds":
        lds(a.counter_csv, a.out_md, a.command)
    elif a.what == "clock":
        clock(a.counter_csv, a.agent_csv, a.bench_json, a.out_md, a.command)
    elif a.what == "kernel-stats":
        kernel_stats(a.stats_csv, a.bench_json, a.out_md, a.command)
    else:
        traffic(a.fetch_csv, a.write_csv, a.bench_json, a.out_json, a.command)
    return 0


if __name__ == "__main__":
    sys.exit(main())
