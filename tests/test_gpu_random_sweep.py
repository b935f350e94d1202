"""A seeded random sweep of the GPU path against the CPU oracle: shapes, leading dimensions, input
and output types, and every kernel of the tables forced through the configuration override (or the
built-in choice), with the persistent mode, grid, split count and streaming hint drawn at random.

Operands are small integers, so every fp32 partial sum is exact and each case must equal the oracle
bit for bit; the ldc padding of C, filled with NaN before the run, must come back untouched. A further
100 cases of the same draw take N(0,1)/sqrt(K) operands and are held to the oracle's tolerance. Each
case is a test of its own, named by its index; the index seeds its draw, so a failure can be rerun
alone with the same inputs.
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import software_pipelined_tiled_amd as spt  # noqa: E402
from gpu_helpers import check_full, run_gpu  # noqa: E402

# (bm, bn, bk, stages, waves, mfma, load path) of every kernel the library builds
KERNELS = [
    (256, 256, 64, 2, 4, 16, 0), (256, 256, 64, 5, 4, 16, 0), (256, 256, 32, 4, 4, 16, 0), (256, 256, 64, 1, 4, 16, 0),
    (256, 128, 64, 3, 4, 16, 0), (256, 128, 64, 2, 4, 16, 0), (256, 128, 64, 1, 4, 16, 0),
    (128, 128, 64, 4, 4, 16, 0), (128, 128, 64, 3, 4, 16, 0), (128, 128, 64, 2, 4, 16, 0), (128, 128, 64, 1, 4, 16, 0),
    (64, 64, 64, 4, 4, 16, 0), (64, 64, 128, 4, 4, 16, 0), (64, 64, 64, 2, 4, 16, 0),
    (32, 32, 128, 4, 2, 16, 0), (32, 32, 128, 8, 2, 16, 0),
    (256, 256, 64, 5, 8, 16, 0), (256, 256, 64, 2, 8, 16, 0), (256, 256, 64, 5, 8, 32, 0),
    (128, 128, 64, 2, 4, 16, 2), (64, 64, 64, 2, 4, 16, 2), (128, 128, 64, 1, 4, 16, 2),
]
N_CASES = 400


def draw_dim(rng, hi):
    """Sizes around the tile and K-tile multiples, with ragged tails, or anywhere in [1, hi]."""
    if rng.random() < 0.5:
        base = int(rng.choice([32, 64, 128, 256]))
        d = base * int(rng.integers(1, max(2, hi // base + 1))) + int(rng.integers(-9, 10))
        return int(min(max(d, 1), hi))
    return int(rng.integers(1, hi + 1))


def draw_case(i):
    rng = np.random.default_rng(0xC0FFEE + i)
    M, N, K = draw_dim(rng, 1000), draw_dim(rng, 1000), draw_dim(rng, 1100)
    lda = K + (int(rng.integers(0, 10)) if rng.random() < 0.4 else 0)
    ldb = K + (int(rng.integers(0, 10)) if rng.random() < 0.4 else 0)
    ldc = N + (int(rng.integers(1, 6)) if rng.random() < 0.4 else 0)
    in_dt = int(rng.choice([si.F16, si.BF16]))
    out_dt = int(rng.choice([si.F16, si.BF16, si.F32]))
    cfg = None
    if rng.random() < 0.85:
        bm, bn, bk, s, w, mf, path = KERNELS[int(rng.integers(0, len(KERNELS)))]
        persistent = int(rng.choice([0, 1, 1, 2]))
        splits = int(rng.choice([1, 1, 2, 3, 4, 7])) if path == 0 else 1
        stream = int(rng.choice([0, 1, 2])) if (bm, w) == (32, 2) else 0
        cfg = dict(bm=bm, bn=bn, bk=bk, stages=s, waves=w, mfma=mf, persistent=persistent, group_m=int(rng.choice([1, 3, 8])),
                   load_path=path, grid=int(rng.integers(1, 8)) if persistent and rng.random() < 0.5 else 0,
                   lds_bytes=0, splits=splits, stream=stream)
        # the override must be one the library accepts for this shape: drop the queue, then the split,
        # where they are not built for it
        for drop in ({}, {"persistent": 1}, {"persistent": 1, "splits": 1}):
            c = dict(cfg, **drop)
            if spt.gemm_select_config_status(M, N, K, in_dt, in_dt, out_dt, lda, ldb, ldc, config=c) == 0:
                cfg = c
                break
        else:
            cfg = None
    return M, N, K, lda, ldb, ldc, in_dt, out_dt, cfg


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case_bit_exact(case):
    M, N, K, lda, ldb, ldc, in_dt, out_dt, cfg = draw_case(case)
    print(f"case {case}: M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} in={in_dt} out={out_dt} config={cfg}", flush=True)
    a = si.make_matrix(M, K, in_dt, "small_int", 900 + 2 * case, ld=lda)
    b = si.make_matrix(N, K, in_dt, "small_int", 901 + 2 * case, ld=ldb)
    c, desc = run_gpu(a, b, K, in_dt, out_dt, ldc=ldc, config=cfg)
    if cfg is not None:
        for k in ("bm", "bn", "bk", "stages", "waves", "splits", "stream"):
            assert desc[k] == cfg[k], (k, desc, cfg)
    check_full(a, b, K, in_dt, out_dt, c, N, exact=True)
    # nothing written into the ldc padding
    pad = np.asarray(c)[:, N:ldc]
    if out_dt == si.F32:
        assert np.isnan(pad).all()
    else:
        dec = pad.astype(np.uint32)
        exp_all_ones = ((dec >> 10) & 31) == 31 if out_dt == si.F16 else ((dec >> 7) & 255) == 255
        man = dec & (1023 if out_dt == si.F16 else 127)
        assert (exp_all_ones & (man != 0)).all()


N_REAL_CASES = 100


@pytest.mark.parametrize("case", range(N_REAL_CASES))
def test_random_case_real_values_within_tolerance(case):
    # the same draw of shapes and configurations (other seeds), with N(0,1)/sqrt(K) operands: every
    # output within the oracle's bound |C - C_ref| <= 2e-3 (|A||B|^T) + 1 ulp
    M, N, K, lda, ldb, ldc, in_dt, out_dt, cfg = draw_case(10_000 + case)
    print(f"real case {case}: M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} in={in_dt} out={out_dt} config={cfg}",
          flush=True)
    a = si.make_matrix(M, K, in_dt, "normal_scaled", 7000 + 2 * case, ld=lda, k_for_scale=K)
    b = si.make_matrix(N, K, in_dt, "normal_scaled", 7001 + 2 * case, ld=ldb, k_for_scale=K)
    c, _ = run_gpu(a, b, K, in_dt, out_dt, ldc=ldc, config=cfg)
    check_full(a, b, K, in_dt, out_dt, c, N)
