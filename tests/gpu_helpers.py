"""Shared helpers for the GPU parity tests: upload seeded operand bits, run the HIP path through
the C ABI, download the result bits, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import synthetic_inputs as si
from oracle import oracle as orc
import software_pipelined_tiled_amd as spt

TORCH_DT = {si.F16: torch.float16, si.BF16: torch.bfloat16, si.F32: torch.float32}
REL_TOL = 2e-3  # |C - C_ref| <= 2e-3 * (|A|·|B|ᵀ)_ij + 1 ulp of the output type


def to_device(bits: np.ndarray, dtype: int, offset_elems: int = 0) -> torch.Tensor:
    """Upload a [rows, ld] uint16 matrix; with offset_elems > 0 the tensor starts that many
    elements into a larger allocation (to exercise misaligned base pointers)."""
    flat = np.ascontiguousarray(bits).view(np.int16).reshape(-1)
    buf = torch.empty(flat.size + offset_elems + 8, dtype=torch.int16, device="cuda")
    buf[offset_elems:offset_elems + flat.size].copy_(torch.from_numpy(flat))
    t = buf[offset_elems:offset_elems + flat.size].view(TORCH_DT[dtype])
    return t.view(bits.shape)


def run_gpu(a_bits, b_bits, K, in_dtype, out_dtype, ldc=None, config=None, a_off=0, b_off=0, c_sentinel=True):
    """C = A·Bᵀ on the GPU; returns (C as uint16 bits or float32 [M, ldc], plan description)."""
    M, lda = a_bits.shape
    N, ldb = b_bits.shape
    ldc = ldc or N
    A = to_device(a_bits, in_dtype, a_off)
    B = to_device(b_bits, in_dtype, b_off)
    odt = TORCH_DT[out_dtype]
    C = torch.empty((max(M, 1), ldc), dtype=odt, device="cuda")
    if c_sentinel:  # NaN everywhere: anything not written, or written out of bounds, shows up
        C.fill_(float("nan"))
    plan = spt.Plan(M, N, K, TORCH_DT[in_dtype], odt, lda, ldb, ldc, config)
    plan.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr())
    torch.cuda.synchronize()
    desc = plan.describe()
    plan.close()
    out = C[:M].cpu()
    if out_dtype == si.F32:
        return out.numpy(), desc
    return out.view(torch.int16).numpy().view(np.uint16), desc


def check_full(a_bits, b_bits, K, in_dtype, out_dtype, c_gpu, N, exact=False):
    """Compare the [M, N] block of c_gpu with the oracle; return the report."""
    c_ref, s, t = orc.gemm(a_bits, b_bits, K, in_dtype, out_dtype)
    got = np.ascontiguousarray(c_gpu[:, :N])
    if exact:
        if out_dtype == si.F32:
            eq = np.array_equal(got.view(np.uint32), c_ref.view(np.uint32))
        else:
            eq = np.array_equal(got, c_ref)
        if not eq:
            bad = np.argwhere(got.view(np.uint32 if out_dtype == si.F32 else np.uint16) !=
                              c_ref.view(np.uint32 if out_dtype == si.F32 else np.uint16))
            raise AssertionError(f"not bit-exact: {len(bad)} mismatches, first at {bad[:5].tolist()}")
    rep = orc.compare(got, c_ref, t, out_dtype, REL_TOL)
    assert rep["ok"], rep
    return rep


def check_full_blocked(a_bits, b_bits, K, in_dtype, out_dtype, c_gpu, N, max_outputs=1 << 24, log=None):
    """Every output of the [M, N] block of c_gpu against the oracle, computed in row blocks of at
    most ``max_outputs`` outputs so that the oracle's fp64 tolerance sums stay bounded in memory.
    Returns the merged report (worst ratio and its (row, column), outputs checked, failures)."""
    M = a_bits.shape[0]
    rows = max(1, min(M, max_outputs // max(N, 1)))
    merged = {"ok": True, "n": 0, "n_fail": 0, "max_ratio": 0.0, "worst_index": None}
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        c_ref, _, t = orc.gemm(a_bits[r0:r1], b_bits, K, in_dtype, out_dtype, want_s=False)
        rep = orc.compare(np.ascontiguousarray(c_gpu[r0:r1, :N]), c_ref, t, out_dtype, REL_TOL)
        merged["n"] += rep["n"]
        merged["n_fail"] += rep["n_fail"]
        if rep["max_ratio"] >= merged["max_ratio"] and rep["worst_index"] is not None:
            merged["max_ratio"] = rep["max_ratio"]
            merged["worst_index"] = (int(rep["worst_index"][0]) + r0, int(rep["worst_index"][1]))
        if not rep["ok"]:
            merged["ok"] = False
            merged["first_failing_block"] = merged.get("first_failing_block", (r0, r1))
        if log:
            log(f"  rows {r0}..{r1 - 1}: max |err|/tol {rep['max_ratio']:.3g}, failures {rep['n_fail']}")
    assert merged["n"] == M * N
    assert merged["ok"], merged
    return merged
