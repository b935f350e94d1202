"""Python face of the CPU oracle — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module. It loads ``liboracle.so`` (plain C, built with gcc by ``oracle/build.py``)
and never touches the HIP library or the GPU.

The arithmetic lives in ``gemm_oracle.c``: an fp64 triple loop with k ascending, the
side sum T = Σ|a||b|, and one round-to-nearest-even into the output type. This file adds
the acceptance rule used by the parity tests:

    accept C_gpu[i,j]  iff  C_gpu finite whenever C_ref is finite, and
                            |C_gpu − C_ref| ≤ rel · T[i,j] + ulp_out(C_ref[i,j])

with rel = 2e-3 in the parity tests (the stated tolerance for this GEMM); the
ulp is that of the output type at C_ref, floored at the type's smallest subnormal.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F16, BF16, F32 = 0, 1, 2

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        L.oracle_decode_f16.restype = ctypes.c_double
        L.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_bf16.restype = ctypes.c_double
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_encode_f16.restype = ctypes.c_uint16
        L.oracle_encode_f16.argtypes = [ctypes.c_double]
        L.oracle_encode_bf16.restype = ctypes.c_uint16
        L.oracle_encode_bf16.argtypes = [ctypes.c_double]
        L.oracle_encode_f32_generic.restype = ctypes.c_uint32
        L.oracle_encode_f32_generic.argtypes = [ctypes.c_double]
        L.oracle_ulp.restype = ctypes.c_double
        L.oracle_ulp.argtypes = [i32, ctypes.c_double]
        for name in ("oracle_decode_array", "oracle_encode_array", "oracle_ulp_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [i32, i64, vp, vp]
        L.oracle_gemm.restype = i32
        L.oracle_gemm.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, i32, vp, i64, vp, vp, i32]
        L.oracle_gemm_sampled.restype = i32
        L.oracle_gemm_sampled.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, i32, i64, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def decode(dtype: int, bits: np.ndarray) -> np.ndarray:
    """fp16/bf16 bit patterns → float64 (exact), or float32 values → float64."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_decode_array(dtype, b.size, _ptr(b), _ptr(out))
    return out


def encode(dtype: int, x: np.ndarray) -> np.ndarray:
    """float64 → output type, round-to-nearest-even: uint16 bits (f16/bf16) or float32."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32 if dtype == F32 else np.uint16)
    lib().oracle_encode_array(dtype, x.size, _ptr(x), _ptr(out))
    return out


def ulp(dtype: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_ulp_array(dtype, x.size, _ptr(x), _ptr(out))
    return out


def _check_operands(a_bits, b_bits, K):
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] < K or b.shape[1] < K:
        raise ValueError("operands must be 2-D [rows, ld] with ld >= K")
    return a, b


def cpu_share() -> int:
    """Threads the oracle runs on by default: the CPUs this process may use, at most 16 (the
    host-core share of one GPU on a shared GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def gemm(a_bits: np.ndarray, b_bits: np.ndarray, K: int, in_dtype: int, out_dtype: int,
         threads: int | None = None, want_sums: bool = True, want_s: bool = True):
    """Full product C = A·Bᵀ over the first K columns of A[M, lda] and B[N, ldb].

    Returns (C_ref, S, T): C_ref as uint16 bits or float32, dense [M, N]; S and T the float64
    sums (None unless ``want_sums``; S also None when ``want_s`` is false, for callers that
    only need the tolerance scale T).
    """
    a, b = _check_operands(a_bits, b_bits, K)
    M, N = a.shape[0], b.shape[0]
    c = np.empty((M, N), dtype=np.float32 if out_dtype == F32 else np.uint16)
    s = np.empty((M, N), dtype=np.float64) if want_sums and want_s else None
    t = np.empty((M, N), dtype=np.float64) if want_sums else None
    threads = threads or cpu_share()
    rc = lib().oracle_gemm(M, N, K, in_dtype, _ptr(a), a.shape[1], _ptr(b), b.shape[1], out_dtype,
                           _ptr(c), N, _ptr(s) if s is not None else None,
                           _ptr(t) if t is not None else None, threads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return c, s, t


def gemm_sampled(a_bits: np.ndarray, b_bits: np.ndarray, K: int, in_dtype: int, out_dtype: int,
                 ii: np.ndarray, jj: np.ndarray):
    """The same sums for the sampled outputs (ii[q], jj[q]); returns (C_ref[q], S[q], T[q])."""
    a, b = _check_operands(a_bits, b_bits, K)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.size
    c = np.empty(n, dtype=np.float32 if out_dtype == F32 else np.uint16)
    s = np.empty(n, dtype=np.float64)
    t = np.empty(n, dtype=np.float64)
    rc = lib().oracle_gemm_sampled(a.shape[0], b.shape[0], K, in_dtype, _ptr(a), a.shape[1], _ptr(b),
                                   b.shape[1], out_dtype, n, _ptr(ii), _ptr(jj), _ptr(c), _ptr(s), _ptr(t))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_sampled failed ({rc})")
    return c, s, t


def compare(c_test: np.ndarray, c_ref: np.ndarray, t_sum: np.ndarray, out_dtype: int, rel: float) -> dict:
    """Elementwise acceptance test of c_test against the oracle (see module docstring).

    c_test / c_ref are uint16 bits (f16, bf16) or float32 (f32), same shape as t_sum.
    Returns a report with ``ok``, the worst |err|/tol, its index, and failure counts.
    """
    x = decode(out_dtype, c_test).astype(np.float64)
    r = decode(out_dtype, c_ref).astype(np.float64)
    t = np.asarray(t_sum, dtype=np.float64)
    tol = rel * t + ulp(out_dtype, r)
    ref_finite = np.isfinite(r)
    bad_nonfinite = ref_finite & ~np.isfinite(x)
    both_inf_match = ~ref_finite & (x == r)
    with np.errstate(invalid="ignore"):
        err = np.where(ref_finite & np.isfinite(x), np.abs(x - r), 0.0)
    ratio = err / tol
    fail = bad_nonfinite | (ratio > 1.0) | (~ref_finite & ~both_inf_match)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    return {
        "ok": not bool(np.any(fail)),
        "n": int(ratio.size),
        "n_fail": int(np.count_nonzero(fail)),
        "n_nonfinite": int(np.count_nonzero(bad_nonfinite)),
        "max_ratio": float(ratio.reshape(-1)[worst]) if ratio.size else 0.0,
        "worst_index": np.unravel_index(worst, ratio.shape) if ratio.size else None,
        "max_abs_err": float(err.max()) if err.size else 0.0,
    }
