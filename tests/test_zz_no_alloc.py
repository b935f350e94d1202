"""The no-allocation entry point (gemm_run_noalloc) against gemm_plan_create + gemm_run, through
the C ABI: the same built-in plan and kernels must give the same bits. Shapes that use the static
scratch array (a staged operand copy; split-K partial planes; a plan cut in two over staged
operands) and one that uses none, each run twice in a row, the second time with a smaller problem,
so the second call finds the first call's data in the array."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import software_pipelined_tiled_amd as spt  # noqa: E402
from gpu_helpers import TORCH_DT, check_full, to_device  # noqa: E402


def bits(t, out_dt):
    t = t.cpu()
    return t.numpy() if out_dt == si.F32 else t.view(torch.int16).numpy().view(np.uint16)


def run_both(M, N, K, in_dt, out_dt, dist, seed):
    a = si.make_matrix(M, K, in_dt, dist, seed, k_for_scale=K)
    b = si.make_matrix(N, K, in_dt, dist, seed + 1, k_for_scale=K)
    A, B = to_device(a, in_dt), to_device(b, in_dt)
    odt = TORCH_DT[out_dt]
    plan = spt.Plan(M, N, K, TORCH_DT[in_dt], odt)
    ws = plan.workspace_bytes()
    C_ref = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    C_na = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    plan.run_ptrs(A.data_ptr(), B.data_ptr(), C_ref.data_ptr())
    spt.gemm_run_noalloc(M, N, K, in_dt, in_dt, out_dt, K, K, N, A.data_ptr(), B.data_ptr(), C_na.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    plan.close()
    r, g = bits(C_ref, out_dt), bits(C_na, out_dt)
    view = np.uint32 if out_dt == si.F32 else np.uint16
    assert np.array_equal(r.view(view), g.view(view)), f"{M}x{N}x{K}: no-alloc result differs from gemm_run"
    return a, b, g, ws


@pytest.mark.parametrize("big,small,in_dt,out_dt,dist", [
    ((4093, 5119, 3071), (700, 900, 1533), si.F16, si.F16, "uniform"),   # staged copy; the big one cut in two
    ((512, 768, 16384), (256, 256, 8192), si.BF16, si.BF16, "normal_scaled"),  # split-K partial planes
    ((300, 500, 1000), (64, 72, 200), si.F16, si.F32, "uniform"),       # no workspace
])
def test_noalloc_matches_plan_and_run(big, small, in_dt, out_dt, dist):
    M, N, K = big
    _, _, _, ws_big = run_both(M, N, K, in_dt, out_dt, dist, 900 + K)
    M, N, K = small
    a, b, g, ws_small = run_both(M, N, K, in_dt, out_dt, dist, 1900 + K)
    check_full(a, b, K, in_dt, out_dt, g, N)


def test_noalloc_workspace_shapes_use_scratch():
    # the cases above do exercise the scratch array: their plans own workspaces of these kinds
    p = spt.Plan(4093, 5119, 3071, torch.float16, torch.float16)
    assert p.describe()["load_path"] == spt.GEMM_LOAD_STAGED and p.workspace_bytes() > 0
    p.close()
    p = spt.Plan(512, 768, 16384, torch.bfloat16, torch.bfloat16)
    assert p.describe()["splits"] > 1 and p.workspace_bytes() > 0
    p.close()


def test_noalloc_rejects_workspace_beyond_scratch_and_bad_args():
    # K = 8191 (not a multiple of 8): staged copies of 8192 x 8192 operands, 268 MB > 64 MiB
    A = torch.zeros((8192, 8191), dtype=torch.float16, device="cuda")
    C = torch.full((8192, 8192), float("nan"), dtype=torch.float16, device="cuda")
    with pytest.raises(spt.GemmError) as e:
        spt.gemm_run_noalloc(8192, 8192, 8191, si.F16, si.F16, si.F16, 8191, 8191, 8192, A.data_ptr(),
                             A.data_ptr(), C.data_ptr())
    assert e.value.status == spt._lib.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(C).all(), "nothing may be enqueued when the call is rejected"
    lib = spt.lib()
    assert lib.gemm_run_noalloc(8, 8, 8, si.F16, si.F16, si.F16, 4, 8, 8, None, None, None, None) == \
        spt._lib.GEMM_ERR_INVALID
    assert lib.gemm_run_noalloc(0, 8, 8, si.F16, si.F16, si.F16, 8, 8, 8, None, None, None, None) == spt._lib.GEMM_OK
    assert lib.gemm_run_noalloc(8, 8, 8, si.F16, si.F16, si.F16, 8, 8, 8, None, None, None, None) == \
        spt._lib.GEMM_ERR_INVALID


@pytest.mark.parametrize("shape,other,in_dt,out_dt", [
    ((700, 900, 1533), (300, 260, 999), si.F16, si.F16),        # staging copy into the scratch array
    ((512, 768, 16384), (256, 256, 8192), si.BF16, si.F32),     # split-K partial planes in the scratch array
])
def test_noalloc_graph_replay_with_scratch_reused(shape, other, in_dt, out_dt):
    # the callers this entry point is for include work recorded under graph capture. Capture one call,
    # then replay it three times; between replays, eager calls of another shape overwrite the scratch
    # array. Every launch writes the scratch it reads before reading it, so each replay must equal the
    # eager result bit for bit.
    M, N, K = shape
    a = si.make_matrix(M, K, in_dt, "small_int", 77 + K)
    b = si.make_matrix(N, K, in_dt, "small_int", 78 + K)
    A, B = to_device(a, in_dt), to_device(b, in_dt)
    odt = TORCH_DT[out_dt]
    Mo, No, Ko = other
    ao = to_device(si.make_matrix(Mo, Ko, in_dt, "small_int", 79 + Ko), in_dt)
    bo = to_device(si.make_matrix(No, Ko, in_dt, "small_int", 80 + Ko), in_dt)
    Co = torch.empty((Mo, No), dtype=odt, device="cuda")
    C_eager = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    C_graph = torch.full((M, N), float("nan"), dtype=odt, device="cuda")

    def call(Ap, Bp, Cp, m, n, k, stream):
        spt.gemm_run_noalloc(m, n, k, in_dt, in_dt, out_dt, k, k, n, Ap, Bp, Cp, stream)

    s = torch.cuda.current_stream().cuda_stream
    call(A.data_ptr(), B.data_ptr(), C_eager.data_ptr(), M, N, K, s)  # eager, and the device's scratch set up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(A.data_ptr(), B.data_ptr(), C_graph.data_ptr(), M, N, K, torch.cuda.current_stream().cuda_stream)
    want = bits(C_eager, out_dt)
    view = np.uint32 if out_dt == si.F32 else np.uint16
    for rep in range(3):
        call(ao.data_ptr(), bo.data_ptr(), Co.data_ptr(), Mo, No, Ko, s)  # another shape through the scratch
        C_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(C_graph, out_dt).view(view), want.view(view)), f"replay {rep}"
    check_full(a, b, K, in_dt, out_dt, want, N, exact=True)
