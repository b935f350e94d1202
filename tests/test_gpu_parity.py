"""GPU parity of the HIP GEMM against the CPU oracle, through the C ABI.

* Small-integer operands (entries in [-3, 3], K·9 < 2^24) make every fp32 partial sum exact, so
  every kernel configuration (tile, stage count, persistent or not, load path) must match the
  oracle bit for bit: a race on a ring slot, a wrong swizzle or a dropped K-tile shows up as a
  mismatch.
* Real-valued operands (the workloads' distributions) are held to |C - C_ref| <= 2e-3·(|A|·|B|ᵀ)
  + 1 ulp of the output type, elementwise.
* Edge cases: ragged M/N/K, K below and around the stage depth, K = 0, padded leading
  dimensions with NaN padding, misaligned base pointers (register-staged path), and that no
  element outside [0, M) x [0, N) of C is written.
* The full-size workloads run in the configuration the benchmark times and are checked against
  the oracle at every output (the oracle runs in row blocks to bound its memory).
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import software_pipelined_tiled_amd as spt  # noqa: E402
from gpu_helpers import TORCH_DT, check_full, check_full_blocked, run_gpu, to_device  # noqa: E402

DMA_CONFIGS = [(256, 256, 2), (256, 256, 1), (256, 128, 3), (256, 128, 2), (256, 128, 1), (128, 128, 4),
               (128, 128, 3), (128, 128, 2), (128, 128, 1), (64, 64, 4), (64, 64, 2)]
REG_CONFIGS = [(128, 128, 2), (64, 64, 2), (128, 128, 1)]
# (bk, stages, waves) of the 256x256 configurations with their own ring shape: the split ring of
# five operand slots, 32-deep K-tiles with four stages, and the two-wave-group kernel (split ring,
# and two stages)
RING_CONFIGS = [(64, 5, 4), (32, 4, 4), (64, 5, 8), (64, 2, 8)]


def cfg(bm, bn, s, path=spt.GEMM_LOAD_DMA, persistent=1, group_m=8, grid=0, bk=64, waves=4, splits=1, mfma=16,
        stream=0):
    return dict(bm=bm, bn=bn, bk=bk, stages=s, waves=waves, mfma=mfma, persistent=persistent, group_m=group_m,
                load_path=path, grid=grid, lds_bytes=0, splits=splits, stream=stream)


def ring_cfg(bk, s, waves, **kw):
    return cfg(256, 256, s, bk=bk, waves=waves, **kw)


def ints(rows, cols, dtype, seed, ld=None):
    return si.make_matrix(rows, cols, dtype, "small_int", seed, ld=ld)


# ------------------------------------------------------------------------- bit-exact sweeps

@pytest.mark.parametrize("bm,bn,s", DMA_CONFIGS)
@pytest.mark.parametrize("persistent", [1, 0])
def test_dma_configs_bit_exact(bm, bn, s, persistent):
    # 3 x 2 tiles of (bm, bn) with ragged edges, K spanning several K-tiles plus a partial one
    M, N, K = 2 * bm + bm // 2 + 3, 2 * bn - 5, 5 * 64 + 16
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, 100 + bm + s)
        b = ints(N, K, in_dt, 200 + bn + s)
        # a small grid forces several rounds of the persistent loop
        c, desc = run_gpu(a, b, K, in_dt, si.F32, config=cfg(bm, bn, s, persistent=persistent,
                                                            grid=3 if persistent else 0))
        assert desc["bm"] == bm and desc["stages"] == s and desc["load_path"] == spt.GEMM_LOAD_DMA
        check_full(a, b, K, in_dt, si.F32, c, N, exact=True)


@pytest.mark.parametrize("bk,s,waves", RING_CONFIGS)
@pytest.mark.parametrize("persistent", [1, 0])
def test_ring_configs_bit_exact(bk, s, waves, persistent):
    # 2 x 2 tiles with ragged edges; K spans several K-tiles plus a partial one
    M, N, K = 256 + 131, 512 - 37, 7 * 64 + 24
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, 500 + bk + s + waves)
        b = ints(N, K, in_dt, 600 + bk + s + waves)
        c, desc = run_gpu(a, b, K, in_dt, si.F32,
                          config=ring_cfg(bk, s, waves, persistent=persistent, grid=3 if persistent else 0))
        assert (desc["bk"], desc["stages"], desc["waves"]) == (bk, s, waves)
        check_full(a, b, K, in_dt, si.F32, c, N, exact=True)


@pytest.mark.parametrize("K", [8, 64, 72, 128, 136, 192, 256, 320, 648])
@pytest.mark.parametrize("bk,s,waves", RING_CONFIGS)
def test_ring_configs_k_around_depth(K, bk, s, waves):
    # fewer K-tiles than ring slots, about as many, and more; K tails of 8 .. 56 elements
    M, N = 300, 260
    a = ints(M, K, si.BF16, 3 * K + s)
    b = ints(N, K, si.BF16, 3 * K + s + 1)
    c, _ = run_gpu(a, b, K, si.BF16, si.F32, config=ring_cfg(bk, s, waves, grid=2))
    check_full(a, b, K, si.BF16, si.F32, c, N, exact=True)


@pytest.mark.parametrize("K", [8, 64, 72, 136, 200])
@pytest.mark.parametrize("s,mfma", [(5, 16), (2, 16), (5, 32)])
@pytest.mark.parametrize("out_dt", [si.F16, si.BF16])
def test_two_group_16bit_epilogue_across_tiles_at_small_k(K, s, mfma, out_dt):
    # the two-group kernel stores a finished tile in the next tile's first memory phase, its fragment
    # reads spread between the stores (16-bit outputs); with one to four K-tiles per tile and five
    # tiles per workgroup, the stores, reads and loads of neighbouring tiles meet in every phase
    M, N = 600, 560
    in_dt = si.F16 if out_dt == si.F16 else si.BF16
    a = ints(M, K, in_dt, 900 + K + s)
    b = ints(N, K, in_dt, 901 + K + mfma)
    c, desc = run_gpu(a, b, K, in_dt, out_dt, config=ring_cfg(64, s, 8, grid=2, mfma=mfma))
    assert (desc["waves"], desc["stages"], desc["grid"]) == (8, s, 2)
    check_full(a, b, K, in_dt, out_dt, c, N, exact=True)


# (bm, bn, bk, stages) of 4-wave configurations whose ring leaves room for the dynamic queue's slot
QUEUE_CONFIGS = [(256, 256, 64, 2), (256, 128, 64, 3), (128, 128, 64, 4), (64, 64, 64, 4), (64, 64, 128, 4)]


@pytest.mark.parametrize("bm,bn,bk,s", QUEUE_CONFIGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_dynamic_queue_bit_exact(bm, bn, bk, s, splits):
    # persistent = 2: after its first unit each workgroup takes the next free one from an atomic
    # counter. Three workgroups over a ragged 3 x 2 grid (times the K ranges) take many units each;
    # three launches in a row check that each launch leaves the counters at zero for the next
    M, N, K = 2 * bm + bm // 2 + 3, 2 * bn - 5, 9 * bk + 24
    a = ints(M, K, si.BF16, 700 + bm + s + splits)
    b = ints(N, K, si.BF16, 800 + bn + bk + splits)
    A, B = to_device(a, si.BF16), to_device(b, si.BF16)
    conf = cfg(bm, bn, s, bk=bk, persistent=2, grid=3, splits=splits)
    plan = spt.Plan(M, N, K, torch.bfloat16, torch.float32, K, K, N, conf)
    desc = plan.describe()
    assert desc["persistent"] == 2 and desc["grid"] == 3 and desc["splits"] == splits
    assert plan.workspace_bytes() > 0
    ref = None
    for run in range(3):
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        plan.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr())
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        if ref is None:
            check_full(a, b, K, si.BF16, si.F32, got, N, exact=True)
            ref = got
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"run {run}"
    plan.close()


def test_dynamic_queue_rejected_where_not_built():
    M = N = K = 512
    for conf, status in ((ring_cfg(64, 5, 8, persistent=2), spt._lib.GEMM_ERR_UNSUPPORTED),   # two-group kernel
                         (ring_cfg(64, 5, 4, persistent=2), spt._lib.GEMM_ERR_UNSUPPORTED),   # ring fills the LDS
                         (cfg(128, 128, 2, path=spt.GEMM_LOAD_REG, persistent=2), spt._lib.GEMM_ERR_UNSUPPORTED),
                         (cfg(128, 128, 4, persistent=3), spt._lib.GEMM_ERR_INVALID)):
        with pytest.raises(spt.GemmError) as e:
            spt.Plan(M, N, K, torch.float16, torch.float16, config=conf)
        assert e.value.status == status, conf


@pytest.mark.parametrize("K", [8, 120, 128, 136, 384, 512, 520, 5 * 128 + 24])
@pytest.mark.parametrize("persistent", [1, 0])
def test_deep_64_tile_bit_exact(K, persistent):
    # the 64x64 tile with 128-deep K-tiles (two 64-wide LDS groups per K-tile, four stages): fewer
    # K-tiles than stages, about as many, and more; K tails inside the first and the second group;
    # M = 32 as in the skinny workload (half the tile's rows past the edge) and a ragged 3 x 2 grid
    for M, N in ((32, 3 * 64 - 24), (2 * 64 + 37, 2 * 64 - 5)):
        a = ints(M, K, si.F16, 40 + K + M)
        b = ints(N, K, si.F16, 41 + K + N)
        c, desc = run_gpu(a, b, K, si.F16, si.F32,
                          config=cfg(64, 64, 4, bk=128, persistent=persistent, grid=2 if persistent else 0))
        assert (desc["bm"], desc["bk"], desc["stages"]) == (64, 128, 4)
        check_full(a, b, K, si.F16, si.F32, c, N, exact=True)


@pytest.mark.parametrize("K", [8, 128, 136, 512, 896, 1032, 1024 + 8 * 128 + 40])
@pytest.mark.parametrize("s", [4, 8])
@pytest.mark.parametrize("persistent,splits", [(1, 1), (0, 1), (1, 3)])
def test_skinny_32_tile_bit_exact(K, s, persistent, splits):
    # the 32x32 tile with 128-deep K-tiles (two waves; four or eight stages, several reads and loads
    # per MFMA slot): fewer K-tiles than stages, about as many, and more; K tails inside either
    # 64-wide group; M = 32 exactly as in the skinny workload, and a ragged 3 x 2 grid
    for M, N in ((32, 5 * 32 - 9), (2 * 32 + 13, 2 * 32 - 5)):
        a = ints(M, K, si.F16, 60 + K + M + s)
        b = ints(N, K, si.F16, 61 + K + N + s)
        c, desc = run_gpu(a, b, K, si.F16, si.F32,
                          config=cfg(32, 32, s, bk=128, waves=2, persistent=persistent, splits=splits,
                                     grid=2 if persistent else 0))
        assert (desc["bm"], desc["bn"], desc["bk"], desc["stages"], desc["waves"]) == (32, 32, 128, s, 2)
        check_full(a, b, K, si.F16, si.F32, c, N, exact=True)


@pytest.mark.parametrize("K", [136, 1032, 1024 + 8 * 128 + 40])
@pytest.mark.parametrize("s", [4, 8])
@pytest.mark.parametrize("persistent,splits", [(1, 1), (0, 1), (1, 3)])
@pytest.mark.parametrize("stream", [1, 2])
def test_stream_hint_bit_exact(K, s, persistent, splits, stream):
    # the non-temporal hint on A or on B changes where lines are cached, not what is computed:
    # every output equals the oracle's exactly, on the staged path too (K not a multiple of 8)
    for M, N in ((32, 5 * 32 - 9), (2 * 32 + 13, 2 * 32 - 5)):
        for k in (K, K - 3):
            a = ints(M, k, si.F16, 70 + k + M + s)
            b = ints(N, k, si.F16, 71 + k + N + s)
            path = spt.GEMM_LOAD_DMA if k % 8 == 0 else spt.GEMM_LOAD_STAGED
            c, desc = run_gpu(a, b, k, si.F16, si.F32,
                              config=cfg(32, 32, s, bk=128, waves=2, persistent=persistent, splits=splits,
                                         grid=2 if persistent else 0, stream=stream, path=path))
            assert (desc["bm"], desc["stages"], desc["stream"], desc["load_path"]) == (32, s, stream, path)
            check_full(a, b, k, si.F16, si.F32, c, N, exact=True)


def test_stream_hint_auto_on_a():
    # the transpose of the skinny shape: N = 32 columns, so every A tile is read by one workgroup and
    # the built-in plan streams A (128 MiB) with the hint; every output against the oracle
    M, N, K = 8192, 32, 8192
    a = si.make_matrix(M, K, si.F16, "uniform", 0x5A11, ld=K)
    b = si.make_matrix(N, K, si.F16, "uniform", 0x5A12, ld=K)
    c, desc = run_gpu(a, b, K, si.F16, si.F16)
    assert (desc["bm"], desc["bn"], desc["stages"], desc["stream"]) == (32, 32, 8, 1)
    check_full_blocked(a, b, K, si.F16, si.F16, c, N)


@pytest.mark.parametrize("M,N,in_dt,stream", [(32, 8192, si.F16, 2), (8192, 32, si.BF16, 1)])
def test_stream_hint_staged_full(M, N, in_dt, stream):
    # K odd: rows of 8191 elements are copied into rows of 8192 first, then the built-in plan streams
    # the copy of the large operand with the hint through the 8-deep 32x32 ring; every output
    K = 8191
    a = si.make_matrix(M, K, in_dt, "uniform", 0x57A6 + M)
    b = si.make_matrix(N, K, in_dt, "uniform", 0x57A7 + N)
    c, desc = run_gpu(a, b, K, in_dt, in_dt)
    assert (desc["bm"], desc["stages"], desc["load_path"], desc["stream"]) == (32, 8, spt.GEMM_LOAD_STAGED, stream)
    check_full_blocked(a, b, K, in_dt, in_dt, c, N)


@pytest.mark.parametrize("bm,bn,s", REG_CONFIGS)
def test_reg_configs_bit_exact(bm, bn, s):
    M, N, K = 2 * bm + 7, bn + 9, 3 * 64 + 13  # K not a multiple of 8: element-masked tail
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, 300 + bm)
        b = ints(N, K, in_dt, 400 + bn)
        c, desc = run_gpu(a, b, K, in_dt, si.F32, config=cfg(bm, bn, s, path=spt.GEMM_LOAD_REG, grid=5))
        assert desc["load_path"] == spt.GEMM_LOAD_REG
        check_full(a, b, K, in_dt, si.F32, c, N, exact=True)


@pytest.mark.parametrize("out_dt", [si.F16, si.BF16, si.F32])
@pytest.mark.parametrize("in_dt", [si.F16, si.BF16])
def test_output_dtypes_bit_exact(in_dt, out_dt):
    # integer sums up to 9·K = 2880: exact in f32; in f16 above 2048 and in bf16 above 256 they
    # round, and the oracle's single rounding of the exact sum must be reproduced exactly
    M, N, K = 300, 264, 320
    a = ints(M, K, in_dt, 7)
    b = ints(N, K, in_dt, 8)
    for c_cfg in (cfg(256, 256, 2), cfg(128, 128, 4), cfg(128, 128, 2, path=spt.GEMM_LOAD_REG),
                  ring_cfg(64, 5, 8), ring_cfg(64, 5, 4), ring_cfg(64, 5, 8, splits=3), cfg(64, 64, 4, splits=2),
                  ring_cfg(64, 5, 8, mfma=32)):
        c, _ = run_gpu(a, b, K, in_dt, out_dt, config=c_cfg)
        check_full(a, b, K, in_dt, out_dt, c, N, exact=True)


def wide_range_column(rows, K, dtype, seed, emin, emax):
    """[rows, K] bits: column 0 normal values of random sign, exponent field in [emin, emax] and
    random mantissa; every other column zero. A·Bᵀ of two such operands is one product per output,
    exact in fp32, so each output tests the conversion of an fp32 value to the output type."""
    rng = np.random.default_rng(seed)
    mbits = 10 if dtype == si.F16 else 7
    e = rng.integers(emin, emax + 1, rows).astype(np.uint32)
    m = rng.integers(0, 1 << mbits, rows).astype(np.uint32)
    sg = rng.integers(0, 2, rows).astype(np.uint32)
    out = np.zeros((rows, K), np.uint16)
    out[:, 0] = ((sg << 15) | (e << mbits) | m).astype(np.uint16)
    return out


OUTPUT_PATH_CONFIGS = (cfg(256, 256, 2), cfg(128, 128, 4), cfg(128, 128, 2, path=spt.GEMM_LOAD_REG),
                       ring_cfg(64, 5, 8), ring_cfg(64, 5, 4), ring_cfg(64, 5, 8, splits=3),
                       cfg(64, 64, 4, splits=2), ring_cfg(64, 5, 8, mfma=32), cfg(32, 32, 8, bk=128, waves=2, stream=2))


@pytest.mark.parametrize("out_dt", [si.F16, si.BF16, si.F32])
@pytest.mark.parametrize("in_dt", [si.F16, si.BF16])
def test_output_rounding_bit_exact(in_dt, out_dt):
    # products spanning far more than the output's range: f16 outputs overflow to infinity, fall to
    # subnormals and to signed zero; bf16 outputs round 16-bit products to 8 bits, ties included.
    # Every kernel's epilogue (and the split-K reduction) converts each exact fp32 product exactly as
    # the oracle rounds it
    M, N, K = 300, 264, 8
    lo, hi = (1, 30) if in_dt == si.F16 else (127 - 20, 127 + 20)
    a = wide_range_column(M, K, in_dt, 11, lo, hi)
    b = wide_range_column(N, K, in_dt, 12, lo, hi)
    for c_cfg in OUTPUT_PATH_CONFIGS:
        c, _ = run_gpu(a, b, K, in_dt, out_dt, config=c_cfg)
        check_full(a, b, K, in_dt, out_dt, c, N, exact=True)


def test_matmul_plan_cache_is_bounded():
    # 70 distinct shapes through matmul, some with workspaces (staged operands, split K): the cache
    # keeps at most its bound of plans, every result equals the oracle, and an evicted shape plans
    # again and still does
    from software_pipelined_tiled_amd import torch_api
    torch_api._plan_cache.clear()
    cases = []
    for i in range(70):
        M, N, K = 40 + 3 * i, 56 + 5 * (i % 7), (64 if i % 3 else 77) + 8 * (i % 5) + (4096 if i % 10 == 0 else 0)
        a, b = ints(M, K, si.F16, 1000 + i), ints(N, K, si.F16, 2000 + i)
        A, B = to_device(a, si.F16), to_device(b, si.F16)
        C = spt.matmul(A, B, torch.float32)
        assert len(torch_api._plan_cache) <= torch_api._PLAN_CACHE_MAX
        cases.append((a, b, K, N, C))
    torch.cuda.synchronize()
    assert len(torch_api._plan_cache) == torch_api._PLAN_CACHE_MAX
    for a, b, K, N, C in cases:
        check_full(a, b, K, si.F16, si.F32, C.cpu().numpy(), N, exact=True)
    a, b, K, N, _ = cases[0]                       # long evicted: planned again
    C = spt.matmul(to_device(a, si.F16), to_device(b, si.F16), torch.float32)
    torch.cuda.synchronize()
    check_full(a, b, K, si.F16, si.F32, C.cpu().numpy(), N, exact=True)
    torch_api._plan_cache.clear()


def test_binding_rejects_views_the_kernels_would_overrun():
    # a view narrower than the plan's K (A, B) or N (C) with the plan's row stride: the kernels would
    # read or write past it, so the binding refuses it before any launch; the exact views run
    M, N, K = 64, 48, 96
    base_a = torch.zeros((M, K + 32), dtype=torch.float16, device="cuda")
    base_b = torch.zeros((N, K + 32), dtype=torch.float16, device="cuda")
    base_c = torch.full((M, N + 16), 5.0, dtype=torch.float16, device="cuda")
    p = spt.Plan(M, N, K, torch.float16, torch.float16, K + 32, K + 32, N + 16)
    with pytest.raises(ValueError):
        p.run(base_a[:, :K - 1], base_b[:, :K], base_c[:, :N])
    with pytest.raises(ValueError):
        p.run(base_a[:, :K], base_b[:, :K - 8], base_c[:, :N])
    with pytest.raises(ValueError):
        p.run(base_a[:, :K], base_b[:, :K], base_c[:, :N - 1])
    with pytest.raises(ValueError):
        spt.matmul(base_a[:, :K], base_b[:, :K], out=base_c[:, :N - 1])
    p.run(base_a[:, :K], base_b[:, :K], base_c[:, :N])
    torch.cuda.synchronize()
    p.close()
    assert bool((base_c[:, :N] == 0).all()) and bool((base_c[:, N:] == 5.0).all())


def test_concurrent_streams():
    # one plan without a workspace run on four streams at once, each on its own operands; and matmul,
    # which keeps one plan per stream, on two streams at once for a shape that splits K (a workspace).
    # Every result equals the oracle bit for bit
    M, N, K = 520, 392, 648
    plan = spt.Plan(M, N, K, torch.float16, torch.float32)
    assert plan.workspace_bytes() == 0
    streams = [torch.cuda.Stream() for _ in range(4)]
    ops = []
    for i, st in enumerate(streams):
        a, b = ints(M, K, si.F16, 500 + i), ints(N, K, si.F16, 600 + i)
        A, B = to_device(a, si.F16), to_device(b, si.F16)
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ops.append((a, b, A, B, C, st))
    torch.cuda.synchronize()
    for _ in range(3):
        for a, b, A, B, C, st in ops:
            plan.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr(), st.cuda_stream)
    torch.cuda.synchronize()
    for a, b, A, B, C, st in ops:
        check_full(a, b, K, si.F16, si.F32, C.cpu().numpy(), N, exact=True)
    plan.close()
    Ms, Ns, Ks = 256, 256, 8192
    assert spt.Plan(Ms, Ns, Ks, torch.bfloat16, torch.bfloat16).describe()["splits"] > 1
    outs = []
    for i, st in enumerate(streams[:2]):
        a, b = ints(Ms, Ks, si.BF16, 700 + i), ints(Ns, Ks, si.BF16, 800 + i)
        A, B = to_device(a, si.BF16), to_device(b, si.BF16)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            C = spt.matmul(A, B, torch.float32)
        outs.append((a, b, C))
    torch.cuda.synchronize()
    for a, b, C in outs:
        check_full(a, b, Ks, si.BF16, si.F32, C.cpu().numpy(), Ns, exact=True)


@pytest.mark.parametrize("in_dt", [si.F16, si.BF16])
def test_subnormal_inputs_bit_exact(in_dt):
    # A entirely subnormal (exponent field 0, random mantissa and sign) against small integers: the
    # sums are exact in fp32 (bf16 subnormals are fp32 subnormals, so the MFMA must keep denormals),
    # and every kernel family must equal the oracle bit for bit, in fp32 and in the input type
    rng = np.random.default_rng(5)
    M, N, K = 200, 136, 72
    mbits = 10 if in_dt == si.F16 else 7
    a = ((rng.integers(0, 2, (M, K)) << 15) | rng.integers(1, 1 << mbits, (M, K))).astype(np.uint16)
    b = ints(N, K, in_dt, 93)
    for out_dt in (si.F32, in_dt):
        for c_cfg in (None, ring_cfg(64, 5, 8), cfg(128, 128, 4), cfg(32, 32, 8, bk=128, waves=2),
                      cfg(128, 128, 2, path=spt.GEMM_LOAD_REG), ring_cfg(64, 5, 8, splits=3)):
            c, _ = run_gpu(a, b, K, in_dt, out_dt, config=c_cfg)
            check_full(a, b, K, in_dt, out_dt, c, N, exact=True)


@pytest.mark.parametrize("out_dt", [si.F16, si.F32])
def test_nonfinite_inputs_propagate(out_dt):
    # an infinity in A and a NaN in B, among small integers (some zero): the oracle's fp64 sums give
    # NaN where inf meets 0 or the NaN, ±inf along the rest of inf's row, and exact values elsewhere.
    # Every kernel family must give NaN where the oracle does, the same infinity, and the same bits
    M, N, K = 300, 264, 200
    a = ints(M, K, si.F16, 91)
    b = ints(N, K, si.F16, 92)
    a[37, 150] = 0x7C00   # +inf
    b[101, 7] = 0x7E00    # NaN
    c_ref, _, _ = orc.gemm(a, b, K, si.F16, out_dt)
    ref = orc.decode(out_dt, c_ref).astype(np.float64)
    assert np.isnan(ref[:, 101]).all() and np.isinf(ref[37]).sum() > 0 and np.isnan(ref[37]).sum() > 1
    for c_cfg in (None, ring_cfg(64, 5, 8), cfg(128, 128, 4), cfg(32, 32, 8, bk=128, waves=2, stream=2),
                  cfg(128, 128, 2, path=spt.GEMM_LOAD_REG), ring_cfg(64, 5, 8, splits=3), cfg(64, 64, 4, splits=2)):
        c, _ = run_gpu(a, b, K, si.F16, out_dt, config=c_cfg)
        got = orc.decode(out_dt, np.ascontiguousarray(c[:, :N])).astype(np.float64)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), c_cfg
        fin = ~nan
        assert np.array_equal(got[fin], ref[fin]), c_cfg


@pytest.mark.parametrize("K", [1, 8, 63, 64, 65, 127, 128, 129, 200, 256])
@pytest.mark.parametrize("s", [1, 2, 3, 4])
def test_k_around_stage_depth(K, s):
    # fewer K-tiles than stages, exactly S, and S + 1: prologue, drain and the masked K tail
    M, N = 130, 96
    a = ints(M, K, si.BF16, K)
    b = ints(N, K, si.BF16, K + 1)
    conf = cfg(128, 128, s) if K % 8 == 0 else cfg(128, 128, 2, path=spt.GEMM_LOAD_REG)
    c, _ = run_gpu(a, b, K, si.BF16, si.F32, config=conf)
    check_full(a, b, K, si.BF16, si.F32, c, N, exact=True)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 33, 65), (255, 257, 63), (256, 256, 256), (8, 8, 8),
                                   (300, 200, 72), (1, 300, 64), (300, 1, 64), (64, 64, 4096)])
def test_edge_shapes_auto_config(M, N, K):
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, M + 3 * N)
        b = ints(N, K, in_dt, N + 5 * K)
        c, _ = run_gpu(a, b, K, in_dt, si.F32)
        check_full(a, b, K, in_dt, si.F32, c, N, exact=True)


def test_k_zero_writes_zeros():
    for conf in (None, cfg(64, 64, 2, path=spt.GEMM_LOAD_REG)):
        a = np.zeros((70, 8), np.uint16)
        b = np.zeros((40, 8), np.uint16)
        c, _ = run_gpu(a, b, 0, si.F16, si.F16, config=conf)
        assert np.all(c[:, :40] == 0)


@pytest.mark.parametrize("conf", [
    cfg(128, 128, 4, group_m=1 << 30),                     # band taller than the grid: clamped to its rows
    cfg(128, 128, 4, group_m=1 << 30, persistent=0),
    cfg(128, 128, 4, grid=1),                              # one workgroup walks every tile
    cfg(128, 128, 4, grid=1 << 30),                        # more workgroups than tiles: trimmed
    cfg(256, 256, 5, waves=8, group_m=1 << 30, grid=1),    # the two-group phase stream over every tile
    cfg(256, 256, 5, waves=8, grid=1, splits=3),
    cfg(64, 64, 4, persistent=2, grid=1),                  # dynamic queue with a single workgroup
])
def test_override_extremes_bit_exact(conf):
    M, N, K = 700, 900, 448
    a = si.make_matrix(M, K, si.BF16, "small_int", 41)
    b = si.make_matrix(N, K, si.BF16, "small_int", 42)
    c, desc = run_gpu(a, b, K, si.BF16, si.BF16, config=conf)
    check_full(a, b, K, si.BF16, si.BF16, c, N, exact=True)
    assert 1 <= desc["group_m"] <= -(-M // conf["bm"]) and desc["grid"] >= 1


def test_run_rejects_null_operands():
    # a null A, B or C for a non-empty problem is GEMM_ERR_INVALID from both entry points, before any
    # launch; with K = 0 the operands are not read, so only C is required (it is zeroed)
    lib = spt.lib()
    M, N, K = 64, 48, 64
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    p = spt.Plan(M, N, K, torch.float16, torch.float16)
    for a, b, c in ((None, B.data_ptr(), C.data_ptr()), (A.data_ptr(), None, C.data_ptr()), (A.data_ptr(), B.data_ptr(), None)):
        assert lib.gemm_run(p.handle, a, b, c, None) == spt._lib.GEMM_ERR_INVALID
        assert lib.gemm_run_noalloc(M, N, K, 0, 0, 0, K, K, N, a, b, c, None) == spt._lib.GEMM_ERR_INVALID
    p.close()
    p0 = spt.Plan(M, N, 0, torch.float16, torch.float16, lda=1, ldb=1, ldc=N)
    assert lib.gemm_run(p0.handle, None, None, C.data_ptr(), None) == 0
    torch.cuda.synchronize()
    p0.close()
    assert bool((C == 0).all())


def test_empty_output_is_a_no_op():
    # M or N = 0 with K > 0: plan creation and the run succeed and write nothing (a regression: the
    # split choice divided by the zero tile count), through the plan and the no-allocation entry point
    K = 64
    for M, N in ((0, 37), (37, 0), (0, 0)):
        A = torch.ones((max(M, 1), K), dtype=torch.float16, device="cuda")
        B = torch.ones((max(N, 1), K), dtype=torch.float16, device="cuda")
        C = torch.full((max(M, 1), max(N, 1)), 7.0, dtype=torch.float16, device="cuda")
        p = spt.Plan(M, N, K, torch.float16, torch.float16, lda=K, ldb=K, ldc=max(N, 1))
        p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr())
        st = spt.lib().gemm_run_noalloc(M, N, K, 0, 0, 0, K, K, max(N, 1), A.data_ptr(), B.data_ptr(),
                                        C.data_ptr(), None)
        torch.cuda.synchronize()
        p.close()
        assert st == 0
        assert bool((C == 7.0).all()), (M, N)


def test_padded_ld_and_no_out_of_bounds_writes():
    M, N, K = 200, 136, 192
    for in_dt in (si.F16, si.BF16):
        # NaN in the A/B padding: reading it would poison the sums
        a = si.make_matrix(M, K, in_dt, "small_int", 21, ld=K + 64, pad_bits=0x7E00 if in_dt == si.F16 else 0x7FC0)
        b = si.make_matrix(N, K, in_dt, "small_int", 22, ld=K + 8, pad_bits=0x7E00 if in_dt == si.F16 else 0x7FC0)
        for out_dt in (si.F16, si.F32):
            ldc = N + 24
            c, desc = run_gpu(a, b, K, in_dt, out_dt, ldc=ldc)
            assert desc["load_path"] == spt.GEMM_LOAD_DMA
            check_full(a, b, K, in_dt, out_dt, c, N, exact=True)
            pad = orc.decode(out_dt, c[:, N:])
            assert np.all(np.isnan(pad)), "the ldc padding of C was written"


def test_misaligned_pointers_use_register_path():
    M, N, K = 150, 120, 128
    a = ints(M, K, si.F16, 31)
    b = ints(N, K, si.F16, 32)
    c, desc = run_gpu(a, b, K, si.F16, si.F32, a_off=1, b_off=3)
    check_full(a, b, K, si.F16, si.F32, c, N, exact=True)


@pytest.mark.parametrize("conf,out_dt", [
    (cfg(256, 256, 5, waves=8), si.BF16),                     # the two-group kernel
    (None, si.BF16),                                          # the built-in choice (32x32 ring tiles)
    (cfg(128, 128, 4), si.BF16),                              # the ring kernel
    (cfg(64, 64, 2, path=spt.GEMM_LOAD_REG), si.F16),         # the register-staged kernel
    (cfg(256, 256, 5, waves=8, splits=3), si.BF16),           # split K: the reduction writes C
    (None, si.F32),
])
@pytest.mark.parametrize("c_off", [1, 3])
def test_misaligned_output_pointer(conf, out_dt, c_off):
    # C's base 2 (f16/bf16) or 4 (f32) bytes off a 16-byte boundary, inside a larger NaN-filled
    # buffer: every output equals the oracle and nothing before or after C, or in its ldc padding,
    # is written
    M, N, K, ldc = 520, 300, 192, 310
    a = ints(M, K, si.BF16 if out_dt != si.F16 else si.F16, 71)
    b = ints(N, K, si.BF16 if out_dt != si.F16 else si.F16, 72)
    in_dt = si.BF16 if out_dt != si.F16 else si.F16
    A, B = to_device(a, in_dt), to_device(b, in_dt)
    odt = TORCH_DT[out_dt]
    guard = 128                                               # elements before C (more than 16 bytes)
    buf = torch.full((guard + c_off + M * ldc + guard,), float("nan"), dtype=odt, device="cuda")
    C = buf[guard + c_off: guard + c_off + M * ldc].view(M, ldc)
    assert C.data_ptr() % 16 != 0
    p = spt.Plan(M, N, K, TORCH_DT[in_dt], odt, K, K, ldc, conf)
    p.run_ptrs(A.data_ptr(), B.data_ptr(), C.data_ptr())
    torch.cuda.synchronize()
    p.close()
    out = C.cpu()
    got = out.numpy() if out_dt == si.F32 else out.view(torch.int16).numpy().view(np.uint16)
    check_full(a, b, K, in_dt, out_dt, got, N, exact=True)
    rest = torch.cat([buf[:guard + c_off], buf[guard + c_off + M * ldc:], C[:, N:].reshape(-1)])
    assert bool(torch.isnan(rest.float()).all()), "written outside C"


def test_a_and_b_may_be_one_matrix():
    # C = A·Aᵀ with both operand pointers on one allocation, through the two-group kernel, the
    # built-in choice and a split-K plan: the result is the oracle's, bit for bit
    M, K = 600, 320
    a = ints(M, K, si.BF16, 81)
    A = to_device(a, si.BF16)
    for conf in (cfg(256, 256, 5, waves=8), None, cfg(256, 256, 5, waves=8, splits=2)):
        C = torch.empty((M, M), dtype=torch.float32, device="cuda")
        p = spt.Plan(M, M, K, torch.bfloat16, torch.float32, K, K, M, conf)
        p.run_ptrs(A.data_ptr(), A.data_ptr(), C.data_ptr())
        torch.cuda.synchronize()
        p.close()
        check_full(a, a, K, si.BF16, si.F32, C.cpu().numpy(), M, exact=True)


def test_deterministic_and_grouping_invariant():
    M, N, K = 520, 700, 448
    a = si.make_matrix(M, K, si.BF16, "normal_scaled", 41, k_for_scale=K)
    b = si.make_matrix(N, K, si.BF16, "normal_scaled", 42, k_for_scale=K)
    c1, _ = run_gpu(a, b, K, si.BF16, si.BF16, config=cfg(128, 128, 4, group_m=8))
    c2, _ = run_gpu(a, b, K, si.BF16, si.BF16, config=cfg(128, 128, 4, group_m=8))
    c3, _ = run_gpu(a, b, K, si.BF16, si.BF16, config=cfg(128, 128, 4, group_m=1, persistent=0))
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)  # tile order does not change any sum
    check_full(a, b, K, si.BF16, si.BF16, c1, N)


# ------------------------------------------------------------------------- 32x32x16 MFMA

@pytest.mark.parametrize("persistent", [1, 0])
@pytest.mark.parametrize("M,N,K", [(256 + 131, 512 - 37, 7 * 64 + 24), (256, 256, 64), (1, 300, 8), (513, 257, 520)])
def test_mfma32_bit_exact(M, N, K, persistent):
    # the two-group kernel on v_mfma_f32_32x32x16: its own fragment rows, B-row order and epilogue
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, 1100 + M + K)
        b = ints(N, K, in_dt, 1200 + N + K)
        for out_dt in (si.F32, si.BF16):
            c, desc = run_gpu(a, b, K, in_dt, out_dt,
                              config=ring_cfg(64, 5, 8, mfma=32, persistent=persistent, grid=3 if persistent else 0))
            assert desc["mfma"] == 32
            check_full(a, b, K, in_dt, out_dt, c, N, exact=True)


def test_mfma32_split_k_and_real_values():
    M, N, K = 300, 700, 4096
    a = ints(M, K, si.BF16, 1301)
    b = ints(N, K, si.BF16, 1302)
    c, _ = run_gpu(a, b, K, si.BF16, si.F32, config=ring_cfg(64, 5, 8, mfma=32, splits=3))
    check_full(a, b, K, si.BF16, si.F32, c, N, exact=True)
    a = si.make_matrix(M, K, si.BF16, "normal_scaled", 1303, k_for_scale=K)
    b = si.make_matrix(N, K, si.BF16, "normal_scaled", 1304, k_for_scale=K)
    c, _ = run_gpu(a, b, K, si.BF16, si.BF16, config=ring_cfg(64, 5, 8, mfma=32))
    check_full(a, b, K, si.BF16, si.BF16, c, N)


# ------------------------------------------------------------------------- split-K and staging

# (bm, bn, bk, stages, waves) of every mainloop kernel that runs split-K units
SPLIT_CONFIGS = [(64, 64, 64, 4, 4), (64, 64, 128, 4, 4), (128, 128, 64, 4, 4), (256, 128, 64, 3, 4),
                 (256, 256, 64, 2, 4), (256, 256, 64, 5, 4), (256, 256, 32, 4, 4), (256, 256, 64, 5, 8),
                 (256, 256, 64, 2, 8)]


@pytest.mark.parametrize("bm,bn,bk,s,waves", SPLIT_CONFIGS)
@pytest.mark.parametrize("splits", [2, 3, 5])
def test_split_k_bit_exact(bm, bn, bk, s, waves, splits):
    # ragged 2 x 2 tiles; 13 K-tiles of 64 (26 of 32) plus a tail, cut into ranges of unequal use
    M, N, K = bm + bm // 2 + 5, 2 * bn - 9, 13 * 64 + 40
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, 900 + bm + s + splits)
        b = ints(N, K, in_dt, 950 + bn + waves + splits)
        for grid in (0, 3):
            c, desc = run_gpu(a, b, K, in_dt, si.F32,
                              config=cfg(bm, bn, s, bk=bk, waves=waves, splits=splits, grid=grid))
            assert desc["splits"] == splits
            check_full(a, b, K, in_dt, si.F32, c, N, exact=True)


@pytest.mark.parametrize("K,splits", [(64, 2), (320, 4), (320, 6), (8, 3), (136, 16), (1000, 7)])
def test_split_k_uneven_and_empty_ranges(K, splits):
    # K-tiles not a multiple of the ranges; with more ranges than K-tiles the last ones are empty
    # and must contribute zeros
    M, N = 100, 140
    for conf in (cfg(64, 64, 4, splits=splits), ring_cfg(64, 5, 8, splits=splits)):
        a = ints(M, K, si.BF16, K + splits)
        b = ints(N, K, si.BF16, K + 2 * splits)
        for out_dt in (si.BF16, si.F32):
            c, _ = run_gpu(a, b, K, si.BF16, out_dt, config=conf)
            check_full(a, b, K, si.BF16, out_dt, c, N, exact=True)


def test_split_k_padded_ldc_and_no_out_of_bounds_writes():
    M, N, K = 130, 75, 2048
    a = ints(M, K, si.F16, 61)
    b = ints(N, K, si.F16, 62)
    for out_dt in (si.F16, si.F32):
        ldc = N + 13  # odd row length: the reduction's unaligned-row stores
        c, desc = run_gpu(a, b, K, si.F16, out_dt, ldc=ldc, config=cfg(64, 64, 4, splits=4))
        assert desc["splits"] == 4
        check_full(a, b, K, si.F16, out_dt, c, N, exact=True)
        pad = orc.decode(out_dt, c[:, N:]) if out_dt != si.F32 else c[:, N:]
        assert np.all(np.isnan(pad)), "the ldc padding of C was written"


def test_split_k_real_values_deterministic():
    M, N, K = 96, 1000, 8192
    a = si.make_matrix(M, K, si.F16, "uniform", 71)
    b = si.make_matrix(N, K, si.F16, "uniform", 72)
    conf = cfg(64, 64, 4, splits=8)
    c1, _ = run_gpu(a, b, K, si.F16, si.F16, config=conf)
    c2, _ = run_gpu(a, b, K, si.F16, si.F16, config=conf)
    assert np.array_equal(c1, c2)  # the ranges are added in a fixed order
    check_full(a, b, K, si.F16, si.F16, c1, N)


@pytest.mark.parametrize("M,N,K,lda,ldb", [(200, 130, 77, 77, 77), (70, 300, 3071, 3071, 3075),
                                           (257, 33, 1, 1, 1), (64, 64, 200, 203, 200), (33, 65, 24, 25, 24)])
def test_staged_operands_bit_exact(M, N, K, lda, ldb):
    # K or a leading dimension not a multiple of 8 (rows only 2-byte aligned): the staged path
    for in_dt in (si.F16, si.BF16):
        a = ints(M, K, in_dt, M + K, ld=lda)
        b = ints(N, K, in_dt, N + K, ld=ldb)
        c, desc = run_gpu(a, b, K, in_dt, si.F32)
        assert desc["load_path"] == spt.GEMM_LOAD_STAGED
        check_full(a, b, K, in_dt, si.F32, c, N, exact=True)
        # the same through explicit kernels, with split K and misaligned base pointers
        for conf in (cfg(128, 128, 4, path=spt.GEMM_LOAD_STAGED), ring_cfg(64, 5, 8, path=spt.GEMM_LOAD_STAGED),
                     cfg(64, 64, 4, path=spt.GEMM_LOAD_STAGED, splits=3)):
            c, desc = run_gpu(a, b, K, in_dt, si.BF16, config=conf, a_off=1, b_off=3)
            assert desc["load_path"] == spt.GEMM_LOAD_STAGED
            check_full(a, b, K, in_dt, si.BF16, c, N, exact=True)


@pytest.mark.parametrize("shape,config,lda", [
    ((256, 256, 256), None, None),                                      # one kernel (deep 64x64 tile)
    ((300, 260, 648), cfg(64, 64, 4, splits=3), None),                  # mainloop + reduction
    ((200, 130, 77), None, 77),                                         # staging copy + mainloop
    ((4096, 5119, 1024), None, None),                                   # two parts, two mainloops
    ((700, 500, 648), cfg(128, 128, 4, persistent=2, grid=5), None),    # dynamic unit queue
])
def test_graph_replay_matches_eager(shape, config, lda):
    # gemm_run captured in a HIP graph and replayed three times, with eager work of the same plan and
    # synchronisations in between; every replay must equal the eager result bit for bit
    M, N, K = shape
    a = ints(M, K, si.F16, 61 + K, ld=lda)
    b = ints(N, K, si.F16, 62 + K, ld=lda)
    A = to_device(a, si.F16)
    B = to_device(b, si.F16)
    plan = spt.Plan(M, N, K, torch.float16, torch.float32, a.shape[1], b.shape[1], N, config)
    C_eager = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C_graph = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    C_other = torch.empty((M, N), dtype=torch.float32, device="cuda")
    plan.run_ptrs(A.data_ptr(), B.data_ptr(), C_eager.data_ptr())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run_ptrs(A.data_ptr(), B.data_ptr(), C_graph.data_ptr(), torch.cuda.current_stream().cuda_stream)
    want = C_eager.cpu()
    for rep in range(3):
        C_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C_graph.cpu().view(torch.int32), want.view(torch.int32)), f"replay {rep}"
        plan.run_ptrs(A.data_ptr(), B.data_ptr(), C_other.data_ptr())  # eager work between replays
        torch.cuda.synchronize()
    plan.close()
    if M * N * K <= 1 << 26:  # the eager result itself, against the oracle (other tests cover the large plan)
        check_full(a, b, K, si.F16, si.F32, want.numpy(), N, exact=True)


def test_spans_beyond_2gib_exact():
    # A spans 2.15 GB (16384 rows of lda = 65600) and the fp32 C 2.68 GB (16384 x 40960): tile base
    # addresses lie past 2^31 bytes while each tile's own offsets stay below it. Integer inputs make
    # every output exact, so every output is compared bit for bit (in row blocks); the NaN sentinel
    # shows any output left unwritten
    M, N, K, lda = 16384, 40960, 64, 65600
    a = ints(M, K, si.BF16, 77, ld=lda)
    b = ints(N, K, si.BF16, 78)
    c, desc = run_gpu(a, b, K, si.BF16, si.F32)
    assert desc["load_path"] == spt.GEMM_LOAD_DMA
    rows = 1024
    for r0 in range(0, M, rows):
        c_ref, _, _ = orc.gemm(a[r0:r0 + rows], b, K, si.BF16, si.F32, want_sums=False)
        got = np.ascontiguousarray(c[r0:r0 + rows])
        if not np.array_equal(got.view(np.uint32), c_ref.view(np.uint32)):
            bad = np.argwhere(got.view(np.uint32) != c_ref.view(np.uint32))
            raise AssertionError(f"rows {r0}..: {len(bad)} mismatches, first at {(bad[:5] + [r0, 0]).tolist()}")


@pytest.mark.parametrize("K,lda", [(1024, 1024), (1023, 1023)])
def test_two_part_plan_bit_exact(K, lda):
    # 4096 x 5119 at 256x256 is 16 x 20 = 320 tiles for 256 workgroups: the plan runs columns
    # [0, 4096) as one full round of 256x256 tiles and the other 1023 as a plan of its own (K = 1023
    # with rows of 1023: both parts read the staged copies). Every output, on both sides of the cut,
    # is compared bit for bit.
    M, N = 4096, 5119
    a = ints(M, K, si.F16, 501 + K, ld=lda)
    b = ints(N, K, si.F16, 502 + K, ld=lda)
    plan = spt.Plan(M, N, K, torch.float16, torch.float32, lda, lda, N)
    parts = plan.parts()
    plan.close()
    assert parts["dim"] == 1 and parts["at"] == 4096 and parts["first"]["bm"] == 256
    c, desc = run_gpu(a, b, K, si.F16, si.F32)
    if K % 8:
        assert desc["load_path"] == spt.GEMM_LOAD_STAGED
    c_ref, _, _ = orc.gemm(a, b, K, si.F16, si.F32, want_sums=False)
    got = np.ascontiguousarray(c[:, :N])
    assert np.array_equal(got.view(np.uint32), c_ref.view(np.uint32))


def test_workspace_sizes():
    p = spt.Plan(300, 500, 4096, torch.float16, torch.float16, config=cfg(64, 64, 4, splits=4))
    assert p.workspace_bytes() == 4 * 300 * 504 * 4
    p.close()
    p = spt.Plan(300, 500, 3071, torch.float16, torch.float16)  # staged: A and B rows of 3072
    assert p.describe()["load_path"] == spt.GEMM_LOAD_STAGED
    assert p.workspace_bytes() >= (300 + 500) * 3072 * 2
    p.close()
    p = spt.Plan(4096, 4096, 4096, torch.bfloat16, torch.bfloat16)
    assert p.workspace_bytes() == 0
    p.close()


# ------------------------------------------------------------------------- the workloads

def test_c1_256_f16_to_f32_full():
    m, n, k, a, b, i_dt, o_dt = si.workload_operands("c1_256_f16_f32")
    c, _ = run_gpu(a, b, k, i_dt, o_dt)
    rep = check_full(a, b, k, i_dt, o_dt, c, n)
    print("c1 max |err|/tol", rep["max_ratio"], flush=True)


@pytest.mark.parametrize("name,shape_index", [("c2_4096_f16_f16", 0), ("c3_8192_bf16_bf16", 0),
                                              ("c4_16384x16384x1024_bf16", 0), ("c5_skinny_ragged_f16", 0),
                                              ("c5_skinny_ragged_f16", 1), ("c5_skinny_ragged_f16", 2)])
def test_workload_full(name, shape_index):
    # The full-size workloads in the plan the benchmark times (the built-in choice, tight leading
    # dimensions). One launch into a NaN-filled C is checked against the oracle at every output;
    # four launches back to back into a second NaN-filled C must give the same bits (the benchmark
    # times launches back to back, so a race between launches, or state one launch leaves for the
    # next, would show there).
    m, n, k, a, b, i_dt, o_dt = si.workload_operands(name, shape_index)
    print(f"{name}[{shape_index}] M={m} N={n} K={k}", flush=True)
    A, B = to_device(a, i_dt), to_device(b, i_dt)
    odt = TORCH_DT[o_dt]
    plan = spt.Plan(m, n, k, TORCH_DT[i_dt], odt)
    desc = plan.describe()
    print(f"  plan {desc} parts {plan.parts()['dim']}", flush=True)
    C1 = torch.full((m, n), float("nan"), dtype=odt, device="cuda")
    C2 = torch.full((m, n), float("nan"), dtype=odt, device="cuda")
    plan.run_ptrs(A.data_ptr(), B.data_ptr(), C1.data_ptr())
    for _ in range(4):
        plan.run_ptrs(A.data_ptr(), B.data_ptr(), C2.data_ptr())
    torch.cuda.synchronize()
    plan.close()
    as_bits = (lambda t: t.cpu().numpy()) if o_dt == si.F32 else (lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16))
    c1, c2 = as_bits(C1), as_bits(C2)
    del C1, C2
    same = np.array_equal(c1.view(np.uint32), c2.view(np.uint32)) if o_dt == si.F32 else np.array_equal(c1, c2)
    assert same, "repeated launches gave different bits"
    rep = check_full_blocked(a, b, k, i_dt, o_dt, c1, n, log=lambda s: print(s, flush=True))
    print(f"  checked {rep['n']} of {m * n} outputs, max |err|/tol {rep['max_ratio']:.3g} at {rep['worst_index']}",
          flush=True)


def test_workload_c1_small_full_through_each_dma_config():
    m, n, k, a, b, i_dt, o_dt = si.workload_operands("c1_256_f16_f32")
    for bm, bn, s in DMA_CONFIGS:
        c, _ = run_gpu(a, b, k, i_dt, o_dt, config=cfg(bm, bn, s))
        check_full(a, b, k, i_dt, o_dt, c, n)
    for bk, s, waves in RING_CONFIGS:
        c, _ = run_gpu(a, b, k, i_dt, o_dt, config=ring_cfg(bk, s, waves))
        check_full(a, b, k, i_dt, o_dt, c, n)
    c, _ = run_gpu(a, b, k, i_dt, o_dt, config=ring_cfg(64, 5, 8, mfma=32))
    check_full(a, b, k, i_dt, o_dt, c, n)
    c, _ = run_gpu(a, b, k, i_dt, o_dt, config=cfg(64, 64, 4, bk=128))
    check_full(a, b, k, i_dt, o_dt, c, n)
