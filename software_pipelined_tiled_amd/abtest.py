"""Same-GPU comparison of library builds from different revisions of this repository.

    python -m software_pipelined_tiled_amd.abtest build REV OUTDIR
        (CPU) extracts the sources of git revision REV and builds them with that revision's own
        build script; the library lands in OUTDIR/libsptgemm.so, the full revision hash beside it
        in OUTDIR/REVISION.
    python -m software_pipelined_tiled_amd.abtest run LIB [LIB ...] [--rounds R] [--workloads c3,c4,c2]
        (GPU) alternates the libraries, each in a fresh process per round: every process first checks
        its library bit for bit against an fp32 product on small-integer operands (shapes that cover
        the two-group kernel, its split-K and two-part plans, the staged path and the ring kernels)
        and stops at the first mismatch, then times each workload (10 launches untimed, then three
        runs of 10; the best and the mean of the three, TFLOP/s). One line per library and round.

The libraries must share the C ABI of the binding in this tree (the shape of gemm_config_t and the
entry points' signatures). Under this load the clock one GPU holds differs from another's by up to 15 %, so
only builds alternated on one GPU in one sequence say anything about each other.
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import tarfile
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

WORKLOADS = {  # name: (M, N, K, input and output type)
    "c2": (4096, 4096, 4096, "f16"),
    "c3": (8192, 8192, 8192, "bf16"),
    "c4": (16384, 16384, 1024, "bf16"),
    "c5a": (32, 8192, 8192, "f16"),
    "c5b": (4093, 5119, 3071, "f16"),
    "c5c": (8192, 1024, 28672, "f16"),
}
# (M, N, K, input type, output type): the two-group kernel with full and edge tiles and several rounds,
# its split-K form, the staged two-part plan, and the 4-wave ring kernels of the smaller shapes
CHECKS = [(8192, 8192, 8192, "bf16", "bf16"), (16384, 16384, 1024, "bf16", "bf16"), (4096, 4096, 4096, "f16", "f16"),
          (4093, 5119, 3071, "f16", "f16"), (8192, 1024, 28672, "f16", "f16"), (1000, 3000, 777, "bf16", "bf16"),
          (2500, 2300, 1111, "f16", "f32"), (777, 5000, 4160, "bf16", "bf16"), (32, 8192, 8192, "f16", "f16")]


def build(rev: str, outdir: str) -> str:
    full = subprocess.run(["git", "-C", ROOT, "rev-parse", rev], check=True, capture_output=True, text=True).stdout.strip()
    with tempfile.TemporaryDirectory() as tmp:
        tar_path = os.path.join(tmp, "src.tar")
        with open(tar_path, "wb") as f:
            subprocess.run(["git", "-C", ROOT, "archive", "--format=tar", full, "software_pipelined_tiled_amd", "include"],
                           check=True, stdout=f)
        with tarfile.open(tar_path) as t:
            t.extractall(os.path.join(tmp, "tree"))
        subprocess.run([sys.executable, os.path.join(tmp, "tree", "software_pipelined_tiled_amd", "build.py")], check=True)
        os.makedirs(outdir, exist_ok=True)
        lib = os.path.join(outdir, "libsptgemm.so")
        shutil.copyfile(os.path.join(tmp, "tree", "software_pipelined_tiled_amd", "libsptgemm.so"), lib)
    with open(os.path.join(outdir, "REVISION"), "w") as f:
        f.write(full + "\n")
    return lib


def _revision(lib: str) -> str:
    p = os.path.join(os.path.dirname(os.path.abspath(lib)), "REVISION")
    return open(p).read().strip()[:12] if os.path.exists(p) else "tree"


def one(lib: str, workloads: list[str]) -> int:
    """Check, then time, one library in this process. Returns a process exit status."""
    from . import _lib
    _lib.LIB_PATH = os.path.abspath(lib)
    import torch
    from .torch_api import Plan
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    rev = _revision(lib)
    torch.cuda.set_device(0)
    for M, N, K, ti, to in CHECKS:
        g = torch.Generator(device="cuda").manual_seed(M + 3 * N + 7 * K)
        A = torch.randint(-3, 4, (M, K), device="cuda", generator=g).to(dt[ti])
        B = torch.randint(-3, 4, (N, K), device="cuda", generator=g).to(dt[ti])
        C = torch.full((M, N), float("nan"), dtype=dt[to], device="cuda")
        p = Plan(M, N, K, dt[ti], dt[to])
        p.run(A, B, C)
        torch.cuda.synchronize()
        # |sums| <= 9K < 2^24: the fp32 product is exact in any order, and both sides round it once
        ref = (A.float() @ B.float().T).to(dt[to])
        p.close()
        if not torch.equal(C.view(torch.int32 if to == "f32" else torch.int16),
                           ref.view(torch.int32 if to == "f32" else torch.int16)):
            print(json.dumps({"rev": rev, "check": [M, N, K, ti, to], "ok": False}), flush=True)
            return 3
    out = {"rev": rev, "lib": lib, "checked": len(CHECKS)}
    for w in workloads:
        M, N, K, t = WORKLOADS[w]
        g = torch.Generator(device="cuda").manual_seed(0)
        A = (torch.randn(M, K, device="cuda", generator=g) / K ** 0.5).to(dt[t])
        B = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(dt[t])
        C = torch.empty(M, N, dtype=dt[t], device="cuda")
        p = Plan(M, N, K, dt[t], dt[t])
        sp = torch.cuda.current_stream().cuda_stream
        for _ in range(10):
            p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)
        rates = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp)
            e1.record()
            torch.cuda.synchronize()
            rates.append(2.0 * M * N * K * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        p.close()
        out[w] = {"best": round(max(rates), 1), "mean": round(sum(rates) / len(rates), 1)}
    print(json.dumps(out), flush=True)
    return 0


def run(libs: list[str], rounds: int, workloads: list[str], timeout: int = 300) -> int:
    for r in range(rounds):
        for lib in libs:
            print(f"round {r + 1}: {lib}", flush=True)
            cmd = [sys.executable, "-m", "software_pipelined_tiled_amd.abtest", "one", lib, "--workloads", ",".join(workloads)]
            rc = subprocess.run(cmd, cwd=ROOT, timeout=timeout).returncode
            if rc != 0:
                print(f"stopped: {lib} exited with {rc}", flush=True)
                return rc
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    b = sub.add_parser("build")
    b.add_argument("rev"), b.add_argument("outdir")
    r = sub.add_parser("run")
    r.add_argument("libs", nargs="+")
    r.add_argument("--rounds", type=int, default=3)
    r.add_argument("--workloads", default="c3,c4,c2")
    o = sub.add_parser("one")
    o.add_argument("lib")
    o.add_argument("--workloads", default="c3,c4,c2")
    a = ap.parse_args(argv)
    if a.what == "build":
        print(build(a.rev, a.outdir))
        return 0
    ws = [w for w in a.workloads.split(",") if w]
    for w in ws:
        if w not in WORKLOADS:
            raise SystemExit(f"unknown workload {w}; one of {sorted(WORKLOADS)}")
    if a.what == "run":
        return run(a.libs, a.rounds, ws)
    return one(a.lib, ws)


if __name__ == "__main__":
    sys.exit(main())
