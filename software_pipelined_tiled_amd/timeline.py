"""Phase timeline of the two-group kernel, from an instrumented copy of it.

    python -m software_pipelined_tiled_amd.timeline build [OUTDIR]     (CPU; default _tl)
        copies csrc/spt_gemm_pp.hip, adds a timestamp after every workgroup barrier of the phase
        stream (wave 0 of each group, workgroups 0-3, into a device array, with a reader exported as
        spt_timeline_read), and links it with the other objects of the in-tree build into
        OUTDIR/libsptgemm.so. The in-tree build must exist (``build.py``).
    python -m software_pipelined_tiled_amd.timeline run [OUTDIR]       (GPU)
        runs 8192^3 bf16, 16384^2 x 1024 bf16 and 4096^3 f16 through that library and prints, per
        recorded wave, the mean length of a memory and of a compute phase in shader clocks (the
        s_memtime counter), apart for the first K-tile of each output tile, whose memory phases hold
        the previous tile's stores.

The recording workgroups pay for the timestamps (a scalar-memory round trip per phase), and the kernel
ends with its slowest workgroup: the instrumented build measured about 5 % slower than the plain one,
so absolute phase lengths carry that offset while their ratios hold.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SLOTS, DEPTH = 8, 4096

GLOBALS = f"""
// timeline: phase-boundary timestamps of wave 0 of each group in workgroups 0..3
__device__ unsigned long long g_tl_clk[{SLOTS}][{DEPTH}];
__device__ unsigned long long g_tl_rt[{SLOTS}][{DEPTH}];
"""
RECORDER = f"""  const int tl_slot = (blockIdx.x < {SLOTS // 2} && v == 0) ? (int)blockIdx.x * 2 + grp : -1;
  int tl_i = 0;
  auto rec = [&]() SPT_INLINE {{
    if (tl_slot >= 0 && tl_i < {DEPTH} && lane == 0) {{
      g_tl_clk[tl_slot][tl_i] = __builtin_readcyclecounter();
      g_tl_rt[tl_slot][tl_i] = __builtin_amdgcn_s_memrealtime();
    }}
    ++tl_i;
  }};
  rec();
"""
READER = """
extern "C" int spt_timeline_read(void* clk, void* rt) {
  if (hipMemcpyFromSymbol(clk, HIP_SYMBOL(spt::g_tl_clk), sizeof(spt::g_tl_clk)) != hipSuccess) return -1;
  if (hipMemcpyFromSymbol(rt, HIP_SYMBOL(spt::g_tl_rt), sizeof(spt::g_tl_rt)) != hipSuccess) return -1;
  return 0;
}
"""
ANCHOR_NS = "namespace spt {\n"
ANCHOR_WAVE = "  const int m_base = 128 * grp + TM * wm;"
ANCHOR_STREAM = "  if (grp == 0) {"
BARRIER = "barrier_sync();"
EXPECTED_BARRIERS = 8  # G0: prologue, two per K-tile, last; G1: two at the start, two per K-tile


def instrument(src: str) -> str:
    """The kernel source with the recorder added; raises if the source no longer has the expected shape."""
    for a in (ANCHOR_NS, ANCHOR_WAVE, ANCHOR_STREAM):
        if src.count(a) != 1:
            raise ValueError(f"kernel source changed: {a.strip()!r} found {src.count(a)} times")
    src = src.replace(ANCHOR_NS, ANCHOR_NS + GLOBALS, 1)
    line_end = src.index("\n", src.index(ANCHOR_WAVE)) + 1
    src = src[:line_end] + RECORDER + src[line_end:]
    i = src.index(ANCHOR_STREAM)
    head, tail = src[:i], src[i:]
    if tail.count(BARRIER) != EXPECTED_BARRIERS:
        raise ValueError(f"kernel source changed: {tail.count(BARRIER)} barriers in the phase stream")
    return head + tail.replace(BARRIER, BARRIER + " rec();") + READER


def build(outdir: str) -> str:
    from . import build as b
    objs = [os.path.join(b.BUILD_DIR, s + ".o") for s in b.SOURCES if s != "spt_gemm_pp.hip"]
    for o in objs:
        if not os.path.exists(o):
            raise SystemExit(f"{o} missing: build the library first")
    os.makedirs(outdir, exist_ok=True)
    src = os.path.join(outdir, "spt_gemm_pp_timeline.hip")
    with open(os.path.join(b.CSRC, "spt_gemm_pp.hip")) as f:
        text = instrument(f.read())
    with open(src, "w") as f:
        f.write(text)
    obj = os.path.join(outdir, "spt_gemm_pp_timeline.o")
    subprocess.run([b.HIPCC, *b.COMMON, "-c", src, "-o", obj], check=True, capture_output=True)
    lib = os.path.join(outdir, "libsptgemm.so")
    subprocess.run([b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, *objs, "-o", lib], check=True)
    return lib


def run(outdir: str) -> None:
    import numpy as np
    import torch
    from . import _lib
    _lib.LIB_PATH = os.path.abspath(os.path.join(outdir, "libsptgemm.so"))
    from .torch_api import Plan
    L = _lib.lib()
    L.spt_timeline_read.restype = ctypes.c_int
    L.spt_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.set_device(0)
    clk = np.zeros((SLOTS, DEPTH), np.uint64)
    rt = np.zeros((SLOTS, DEPTH), np.uint64)
    shapes = {"c4 16384^2 x 1024 bf16": (16384, 16384, 1024, torch.bfloat16),
              "c3 8192^3 bf16": (8192, 8192, 8192, torch.bfloat16), "c2 4096^3 f16": (4096, 4096, 4096, torch.float16)}
    for name, (M, N, K, dt) in shapes.items():
        g = torch.Generator(device="cuda").manual_seed(0)
        A = (torch.randn(M, K, device="cuda", generator=g) / K ** 0.5).to(dt)
        B = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(dt)
        C = torch.empty(M, N, dtype=dt, device="cuda")
        p = Plan(M, N, K, dt, dt)
        d = p.describe()
        if (d["bm"], d["bn"], d["waves"], d["splits"]) != (256, 256, 8, 1):
            raise SystemExit(f"{name}: the plan is not the two-group kernel: {d}")
        for _ in range(8):
            p.run(A, B, C)
        torch.cuda.synchronize()
        clk[:] = 0
        rt[:] = 0
        if L.spt_timeline_read(clk.ctypes.data, rt.ctypes.data) != 0:
            raise SystemExit("reading the timeline failed")
        p.close()
        KT = (K + 63) // 64
        tiles = -(-(M // 256) * (N // 256) // d["grid"])
        print(f"== {name}: {KT} K-tiles per output tile, {tiles} tiles per workgroup", flush=True)
        for slot in range(SLOTS):
            grp = slot % 2
            # G0 stamps: start, prologue barrier, then (memory end, compute end) per K-tile, last barrier;
            # G1 stamps: start, two barriers, then (memory end, compute end) per K-tile
            first = 2 if grp == 0 else 3
            n = first + 2 * KT * tiles
            c = clk[slot][:n].astype(np.int64)
            r = rt[slot][:n].astype(np.int64)
            if np.any(np.diff(c) <= 0):
                print(f"wg {slot // 2} G{grp}: incomplete record", flush=True)
                continue
            ph = np.diff(c)[first - 1:]
            mem, comp = ph[0::2], ph[1::2]
            start = np.arange(len(mem)) % KT == 0
            ghz = (c[-1] - c[0]) / ((r[-1] - r[0]) * 10.0)
            print(f"wg {slot // 2} G{grp}: {ghz:.2f} GHz; memory phase {mem[~start].mean():.0f} clk, first of a tile "
                  f"{mem[start].mean():.0f}; compute phase {comp[~start].mean():.0f}, first of a tile "
                  f"{comp[start].mean():.0f}; to the first barrier {c[first - 1] - c[0]} clk", flush=True)


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if not argv or argv[0] not in ("build", "run"):
        raise SystemExit(__doc__)
    outdir = argv[1] if len(argv) > 1 else os.path.join(ROOT, "_tl")
    if argv[0] == "build":
        print(build(outdir))
    else:
        run(outdir)
    return 0


if __name__ == "__main__":
    sys.exit(main())
