"""torch-tensor convenience over the C ABI: plans and a ``matmul`` that enqueues on torch's
current stream. torch provides the device memory and the stream handle; all arithmetic runs in
the HIP kernels.
"""
from __future__ import annotations

from collections import OrderedDict

import torch

from . import _lib

_DT = {torch.float16: _lib.GEMM_F16, torch.bfloat16: _lib.GEMM_BF16, torch.float32: _lib.GEMM_F32}


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


class Plan:
    """Owns a gemm_plan_t for C[M,N] = A[M,K]·B[N,K]ᵀ with the given dtypes and leading dimensions."""

    def __init__(self, M, N, K, in_dtype: torch.dtype, out_dtype: torch.dtype, lda=None, ldb=None, ldc=None,
                 config=None):
        self.M, self.N, self.K = int(M), int(N), int(K)
        self.lda = int(lda if lda is not None else K)
        self.ldb = int(ldb if ldb is not None else K)
        self.ldc = int(ldc if ldc is not None else N)
        self.in_dtype, self.out_dtype = in_dtype, out_dtype
        self.handle = None
        self.handle = _lib.gemm_plan_create(self.M, self.N, self.K, dtype_code(in_dtype), dtype_code(in_dtype),
                                            dtype_code(out_dtype), self.lda, self.ldb, self.ldc, config)
        self.device = torch.cuda.current_device()  # where the library made the plan and its workspace

    def describe(self) -> dict:
        return _lib.gemm_plan_describe(self.handle)

    def parts(self) -> dict:
        return _lib.gemm_plan_parts(self.handle)

    def workspace_bytes(self) -> int:
        return _lib.gemm_plan_workspace_bytes(self.handle)

    def run_ptrs(self, a_ptr: int, b_ptr: int, c_ptr: int, stream: int | None = None) -> None:
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        _lib.gemm_run(self.handle, a_ptr, b_ptr, c_ptr, stream)

    def run(self, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream: int | None = None) -> torch.Tensor:
        # the kernels touch rows x cols elements at row stride ld from each base pointer
        for name, t, rows, cols, ld, dt in (("A", A, self.M, self.K, self.lda, self.in_dtype),
                                            ("B", B, self.N, self.K, self.ldb, self.in_dtype),
                                            ("C", C, self.M, self.N, self.ldc, self.out_dtype)):
            if not t.is_cuda or t.dtype != dt:
                raise ValueError(f"{name} must be a {dt} device tensor")
            if t.device.index != self.device:
                raise ValueError(f"{name} is on cuda:{t.device.index}, the plan on cuda:{self.device}")
            if rows > 0 and cols > 0 and (t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols or t.stride(1) != 1
                                          or t.stride(0) != ld):
                raise ValueError(f"{name} must be [>= {rows}, >= {cols}] row-major with row stride {ld}")
        self.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream)
        return C

    def close(self) -> None:
        if self.handle is not None:
            _lib.gemm_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# matmul's plans, least recently used first. A plan may own a device workspace (staged operands up
# to 3 GiB, split-K partial planes up to 1 GiB), so the cache is bounded: the oldest plan is freed
# when a new one would exceed _PLAN_CACHE_MAX, after its device has finished the work it enqueued.
_PLAN_CACHE_MAX = 64
_plan_cache: OrderedDict = OrderedDict()


def _evict_oldest() -> None:
    key, plan = _plan_cache.popitem(last=False)
    torch.cuda.synchronize(key[-2])  # work enqueued with the plan must be done before its workspace goes
    plan.close()


def matmul(A: torch.Tensor, B: torch.Tensor, out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
           config: dict | None = None) -> torch.Tensor:
    """C = A·Bᵀ for device tensors A[M,K], B[N,K] (row-major, unit column stride), on A's device and
    that device's current stream."""
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A[M,K] and B[N,K] required")
    if B.device != A.device or (out is not None and out.device != A.device):
        raise ValueError("A, B and out must be on one device")
    M, K = A.shape
    N = B.shape[0]
    out_dtype = out_dtype or A.dtype
    with torch.cuda.device(A.device):
        C = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=A.device)
        # a plan with a workspace must not run on two streams at once: one cached plan per stream
        stream = torch.cuda.current_stream(A.device).cuda_stream
        key = (M, N, K, A.dtype, out_dtype, A.stride(0), B.stride(0), C.stride(0),
               tuple(sorted(config.items())) if config else None, A.device.index, stream)
        plan = _plan_cache.get(key)
        if plan is None:
            plan = Plan(M, N, K, A.dtype, out_dtype, A.stride(0), B.stride(0), C.stride(0), config)
            while len(_plan_cache) >= _PLAN_CACHE_MAX:
                _evict_oldest()
            _plan_cache[key] = plan
        else:
            _plan_cache.move_to_end(key)
        return plan.run(A, B, C, stream)
