"""ctypes binding of ``libsptgemm.so`` (the C ABI declared in include/gemm.h).

Argument marshalling only: every function forwards to the library entry point of the same
name. Loading fails loudly (``GemmLibraryMissing``) when the library has not been built; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsptgemm.so")

GEMM_F16, GEMM_BF16, GEMM_F32 = 0, 1, 2
GEMM_OK, GEMM_ERR_INVALID, GEMM_ERR_UNSUPPORTED, GEMM_ERR_HIP, GEMM_ERR_NOMEM = 0, -1, -2, -3, -4
GEMM_LOAD_AUTO, GEMM_LOAD_DMA, GEMM_LOAD_REG, GEMM_LOAD_STAGED = 0, 1, 2, 3

# every entry point include/gemm.h declares
EXPORTS = ("gemm_plan_create", "gemm_run", "gemm_run_noalloc", "gemm_plan_destroy", "gemm_plan_describe", "gemm_plan_workspace_bytes",
           "gemm_plan_parts", "gemm_status_string",
           "gemm_select_config", "gemm_select_parts", "gemm_schedule_tile", "gemm_pipeline_protocol", "gemm_lds_chunk_offset", "gemm_probe_mfma_peak",
           "gemm_probe_copy", "gemm_probe_read", "gemm_probe_lds_read")


class GemmLibraryMissing(ImportError):
    pass


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


class GemmConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("bm", "bn", "bk", "stages", "waves", "mfma", "persistent", "group_m",
                                            "load_path", "grid", "lds_bytes", "splits", "stream")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: dict) -> "GemmConfig":
        c = cls()
        for k, v in d.items():
            setattr(c, k, int(v))
        return c


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GemmLibraryMissing(f"{LIB_PATH} is not built; run software_pipelined_tiled_amd/build.py "
                                 "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    P = ctypes.POINTER
    L.gemm_plan_create.restype = i32
    L.gemm_plan_create.argtypes = [P(vp), i64, i64, i64, i32, i32, i32, i64, i64, i64, P(GemmConfig)]
    L.gemm_run.restype = i32
    L.gemm_run.argtypes = [vp, vp, vp, vp, vp]
    L.gemm_run_noalloc.restype = i32
    L.gemm_run_noalloc.argtypes = [i64, i64, i64, i32, i32, i32, i64, i64, i64, vp, vp, vp, vp]
    L.gemm_plan_destroy.restype = i32
    L.gemm_plan_destroy.argtypes = [vp]
    L.gemm_plan_describe.restype = i32
    L.gemm_plan_describe.argtypes = [vp, P(GemmConfig)]
    L.gemm_plan_workspace_bytes.restype = i32
    L.gemm_plan_workspace_bytes.argtypes = [vp, P(i64)]
    L.gemm_plan_parts.restype = i32
    L.gemm_plan_parts.argtypes = [vp, P(i32), P(i64), P(GemmConfig), P(GemmConfig)]
    L.gemm_select_parts.restype = i32
    L.gemm_select_parts.argtypes = [i64, i64, i64, i32, i32, i32, i64, i64, i64, i32, i32, P(i32), P(i64),
                                    P(GemmConfig), P(GemmConfig)]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_status_string.argtypes = [i32]
    L.gemm_select_config.restype = i32
    L.gemm_select_config.argtypes = [i64, i64, i64, i32, i32, i32, i64, i64, i64, i32, i32, P(GemmConfig),
                                     P(GemmConfig)]
    L.gemm_schedule_tile.restype = i32
    L.gemm_schedule_tile.argtypes = [i64, i64, i32, i32, i32, i32, i32, P(i64), P(i64), P(i32)]
    L.gemm_pipeline_protocol.restype = i32
    L.gemm_pipeline_protocol.argtypes = [i32, i32, i32, i32, i32, P(i32), i32]
    L.gemm_lds_chunk_offset.restype = i64
    L.gemm_lds_chunk_offset.argtypes = [i32, i32, i32, i32]
    L.gemm_probe_mfma_peak.restype = i32
    L.gemm_probe_mfma_peak.argtypes = [i64, i32, vp, P(ctypes.c_double)]
    L.gemm_probe_copy.restype = i32
    L.gemm_probe_copy.argtypes = [vp, vp, i64, vp]
    L.gemm_probe_lds_read.restype = i32
    L.gemm_probe_lds_read.argtypes = [i32, i64, vp]
    L.gemm_probe_read.restype = i32
    L.gemm_probe_read.argtypes = [vp, i64, vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gemm_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != GEMM_OK:
        raise GemmError(status, where)


def gemm_plan_create(M: int, N: int, K: int, a_dtype: int, b_dtype: int, c_dtype: int, lda: int, ldb: int,
                     ldc: int, config: GemmConfig | dict | None = None) -> int:
    """Returns the plan handle (an integer pointer). Raises GemmError on a non-OK status."""
    if isinstance(config, dict):
        config = GemmConfig.from_dict(config)
    plan = ctypes.c_void_p()
    st = lib().gemm_plan_create(ctypes.byref(plan), M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc,
                                ctypes.byref(config) if config is not None else None)
    _check(st, "gemm_plan_create")
    return plan.value


def gemm_run(plan: int, a_ptr: int, b_ptr: int, c_ptr: int, stream: int = 0) -> None:
    _check(lib().gemm_run(plan, a_ptr, b_ptr, c_ptr, stream or None), "gemm_run")


def gemm_run_noalloc(M: int, N: int, K: int, a_dtype: int, b_dtype: int, c_dtype: int, lda: int, ldb: int, ldc: int,
                     a_ptr: int, b_ptr: int, c_ptr: int, stream: int = 0) -> None:
    _check(lib().gemm_run_noalloc(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, a_ptr, b_ptr, c_ptr,
                                  stream or None), "gemm_run_noalloc")


def gemm_plan_destroy(plan: int | None) -> None:
    _check(lib().gemm_plan_destroy(plan), "gemm_plan_destroy")


def gemm_plan_describe(plan: int) -> dict:
    c = GemmConfig()
    _check(lib().gemm_plan_describe(plan, ctypes.byref(c)), "gemm_plan_describe")
    return c.as_dict()


def _parts_dict(dim, at, first, second) -> dict:
    d = {"dim": dim.value, "at": at.value, "first": first.as_dict()}
    if dim.value >= 0:
        d["second"] = second.as_dict()
    return d


def gemm_plan_parts(plan: int) -> dict:
    """{'dim': -1 | 0 (rows cut) | 1 (columns cut), 'at': cut position, 'first': config[, 'second': config]}"""
    dim, at, first, second = ctypes.c_int(), ctypes.c_int64(), GemmConfig(), GemmConfig()
    _check(lib().gemm_plan_parts(plan, ctypes.byref(dim), ctypes.byref(at), ctypes.byref(first),
                                 ctypes.byref(second)), "gemm_plan_parts")
    return _parts_dict(dim, at, first, second)


def gemm_select_parts(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count=256, lds_bytes=160 * 1024) -> dict:
    dim, at, first, second = ctypes.c_int(), ctypes.c_int64(), GemmConfig(), GemmConfig()
    _check(lib().gemm_select_parts(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes,
                                   ctypes.byref(dim), ctypes.byref(at), ctypes.byref(first), ctypes.byref(second)),
           "gemm_select_parts")
    return _parts_dict(dim, at, first, second)


def gemm_plan_workspace_bytes(plan: int) -> int:
    n = ctypes.c_int64()
    _check(lib().gemm_plan_workspace_bytes(plan, ctypes.byref(n)), "gemm_plan_workspace_bytes")
    return n.value


def _config_ref(config):
    if config is None:
        return None
    if isinstance(config, dict):
        config = GemmConfig.from_dict(config)
    return ctypes.byref(config)


def gemm_select_config(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count=256, lds_bytes=160 * 1024,
                       config=None) -> dict:
    c = GemmConfig()
    _check(lib().gemm_select_config(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes,
                                    _config_ref(config), ctypes.byref(c)), "gemm_select_config")
    return c.as_dict()


def gemm_select_config_status(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count=256,
                              lds_bytes=160 * 1024, config=None) -> int:
    c = GemmConfig()
    return lib().gemm_select_config(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes,
                                    _config_ref(config), ctypes.byref(c))


def gemm_schedule_tile(tiles_m, tiles_n, splits, group_m, grid, wg, rnd):
    """(tm, tn, split) for workgroup `wg` in round `rnd`, None if it has no unit; raises on invalid args."""
    tm, tn, sp = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    r = lib().gemm_schedule_tile(tiles_m, tiles_n, splits, group_m, grid, wg, rnd, ctypes.byref(tm),
                                 ctypes.byref(tn), ctypes.byref(sp))
    if r < 0:
        raise GemmError(GEMM_ERR_INVALID, "gemm_schedule_tile")
    return (tm.value, tn.value, sp.value) if r == 1 else None


PROTOCOL_FIELDS = ("la", "lb", "lw", "split", "prologue_wait", "handover_wait", "refill_now", "refill_later",
                   "pp_g0_prologue_wait", "pp_g1_wait")


def gemm_pipeline_protocol(bm: int, bn: int, bk: int, stages: int, waves: int) -> dict | None:
    """The kernel's pipeline counts for this shape (None if no DMA kernel has it)."""
    out = (ctypes.c_int * 10)()
    n = lib().gemm_pipeline_protocol(bm, bn, bk, stages, waves, out, 10)
    return dict(zip(PROTOCOL_FIELDS, out)) if n == 10 else None


def gemm_lds_chunk_offset(rows: int, bk: int, row: int, chunk: int) -> int:
    return lib().gemm_lds_chunk_offset(rows, bk, row, chunk)


def gemm_probe_mfma_peak(iters: int, waves_per_simd: int = 2, stream: int = 0) -> float:
    flops = ctypes.c_double()
    _check(lib().gemm_probe_mfma_peak(iters, waves_per_simd, stream or None, ctypes.byref(flops)),
           "gemm_probe_mfma_peak")
    return flops.value


def gemm_probe_copy(src_ptr: int, dst_ptr: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().gemm_probe_copy(src_ptr, dst_ptr, nbytes, stream or None), "gemm_probe_copy")


def gemm_probe_lds_read(swizzle: int, iters: int, stream: int = 0) -> None:
    _check(lib().gemm_probe_lds_read(swizzle, iters, stream or None), "gemm_probe_lds_read")


def gemm_probe_read(src_ptr: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().gemm_probe_read(src_ptr, nbytes, stream or None), "gemm_probe_read")
