"""Pins for the CPU oracle (oracle/gemm_oracle.c), independent of the oracle's own code.

Every check compares the oracle with something it does not share code with: numpy's and
torch's float conversions (library routines), closed forms of the product (all-ones,
identity, permutation and rank-1 operands), and exact int64 products of small-integer
operands. ``test_pins_catch_planted_mistakes`` compiles copies of the oracle with a
plausible mistake planted in them and checks that at least one pin fails for each.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from oracle import oracle as orc
import synthetic_inputs as si

F16, BF16, F32 = orc.F16, orc.BF16, orc.F32
RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------------------- codecs

def pin_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(F16, bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _f16_midpoints():
    v = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0  # exact in float64
    return np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), [65519.0, 65520.0, 65536.0]])


def pin_f16_encode_vs_numpy():
    x = np.concatenate([
        RNG.uniform(-70000, 70000, 200_000),
        RNG.uniform(-1, 1, 200_000),
        RNG.uniform(-2 ** -13, 2 ** -13, 200_000),  # subnormal range
        np.ldexp(RNG.uniform(1, 2, 100_000), RNG.integers(-30, 17, 100_000)),
        _f16_midpoints(), -_f16_midpoints(),
        [0.0, -0.0, np.inf, -np.inf],
    ])
    got = orc.encode(F16, x)
    with np.errstate(over="ignore"):  # values past the f16 range round to infinity, as the encoder must
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]


def pin_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(BF16, bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_bf16_encode_vs_torch():
    # inputs exactly representable in float32, so torch's float32 -> bfloat16 rounding is the
    # single nearest-even rounding of the value itself
    x32 = np.concatenate([
        RNG.uniform(-4, 4, 300_000).astype(np.float32),
        np.ldexp(RNG.uniform(1, 2, 100_000), RNG.integers(-135, 128, 100_000)).astype(np.float32),
    ])
    # midpoints between adjacent bf16 values (9 significant bits: exact in float32)
    hb = np.arange(0x0080, 0x7F7F, 7, dtype=np.uint32)
    lo = (hb << 16).view(np.float32).astype(np.float64)
    hi = ((hb + 1) << 16).view(np.float32).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    x32 = np.concatenate([x32, mids, -mids])
    x32 = x32[np.isfinite(x32)]
    got = orc.encode(BF16, x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]


def pin_bf16_single_rounding():
    # 1 + 2^-8 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-7: one rounding from
    # float64 gives 1 + 2^-7 (0x3F81); rounding through float32 first would give 1.0 (0x3F80).
    assert int(orc.encode(BF16, np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0]) == 0x3F81
    assert int(orc.encode(BF16, np.array([1 + 2.0 ** -8]))[0]) == 0x3F80  # tie -> even
    assert int(orc.encode(BF16, np.array([1 + 3 * 2.0 ** -8]))[0]) == 0x3F82  # tie -> even (up)
    big = (2 - 2.0 ** -8) * 2.0 ** 127  # midpoint above bf16's max finite: ties to even = inf
    assert int(orc.encode(BF16, np.array([big]))[0]) == 0x7F80
    assert int(orc.encode(BF16, np.array([np.nextafter(big, 0)]))[0]) == 0x7F7F


def pin_generic_encoder_vs_c_float_cast():
    lib = orc.lib()
    x = np.concatenate([
        RNG.standard_normal(50_000) * 1e3,
        np.ldexp(RNG.uniform(1, 2, 50_000), RNG.integers(-160, 130, 50_000)),
    ])
    with np.errstate(over="ignore"):  # values past the f32 range round to infinity, as the encoder must
        ref = x.astype(np.float32).view(np.uint32)
    got = np.array([lib.oracle_encode_f32_generic(float(v)) for v in x], dtype=np.uint32)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]
    f32 = orc.encode(F32, x)
    assert np.array_equal(f32.view(np.uint32), ref)


def pin_ulp():
    v = np.arange(1, 0x7BFF, dtype=np.uint32).astype(np.uint16).view(np.float16)
    assert np.array_equal(orc.ulp(F16, v.astype(np.float64)), np.spacing(v).astype(np.float64))
    x32 = np.ldexp(RNG.uniform(1, 2, 20_000), RNG.integers(-148, 127, 20_000)).astype(np.float32)
    assert np.array_equal(orc.ulp(F32, x32.astype(np.float64)), np.spacing(x32).astype(np.float64))
    # bf16: closed form 2^(e-7), subnormal quantum 2^-133
    assert orc.ulp(BF16, np.array([1.0, 1.5, 2.0, 3.9, 2.0 ** -126, 2.0 ** -130, 0.0])).tolist() == \
        [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133]
    assert orc.ulp(F16, np.array([0.0]))[0] == 2.0 ** -24
    assert orc.ulp(F32, np.array([0.0]))[0] == 2.0 ** -149


# ----------------------------------------------------------------------------- the product

def _bits(dtype, x):
    return si.to_f16_bits(np.asarray(x, np.float64)) if dtype == F16 else si.to_bf16_bits(np.asarray(x, np.float64))


def pin_ones_closed_form():
    for dtype, out, K, expect in [(F16, F16, 3071, 3072.0), (F16, F32, 3071, 3071.0), (BF16, BF16, 1000, 1000.0),
                                  (BF16, BF16, 1001, 1000.0), (BF16, BF16, 1003, 1004.0),
                                  (BF16, BF16, 1002, 1000.0), (BF16, BF16, 1006, 1008.0),  # ties to even
                                  (F16, F16, 100, 100.0)]:
        a = _bits(dtype, np.ones((3, K)))
        b = _bits(dtype, np.ones((5, K)))
        c, s, t = orc.gemm(a, b, K, dtype, out)
        assert np.all(orc.decode(out, c) == expect), (dtype, out, K)
        assert np.all(s == K) and np.all(t == K)


def pin_identity_and_permutation():
    for dtype in (F16, BF16):
        M, K = 7, 24
        a = si.make_matrix(M, K, dtype, "uniform", 99)
        eye = _bits(dtype, np.eye(K))
        for out in (dtype, F32):
            c, s, _ = orc.gemm(a, eye, K, dtype, out)
            assert np.array_equal(orc.decode(out, c), orc.decode(dtype, a)), (dtype, out)
        perm = RNG.permutation(K)
        p = np.zeros((K, K))
        p[np.arange(K), perm] = 1.0  # row j of B selects column perm[j] of A
        c, s, _ = orc.gemm(a, _bits(dtype, p), K, dtype, F32)
        assert np.array_equal(s, orc.decode(dtype, a)[:, perm])


def pin_rank1():
    # K = 1: outer product, rounded once
    for dtype, out in [(F16, F16), (BF16, BF16), (F16, F32)]:
        a = si.make_matrix(9, 1, dtype, "uniform", 5)
        b = si.make_matrix(11, 1, dtype, "uniform", 6)
        c, s, t = orc.gemm(a, b, 1, dtype, out)
        outer = np.outer(orc.decode(dtype, a)[:, 0], orc.decode(dtype, b)[:, 0])
        assert np.array_equal(s, outer)
        assert np.array_equal(t, np.abs(outer))
        ref = outer.astype(np.float32) if out == F32 else (outer.astype(np.float16).view(np.uint16) if out == F16
                                                          else None)
        if ref is not None:
            assert np.array_equal(c, ref)
    # A = u vᵀ, B = w vᵀ with v in {±1}^K  ->  S = K u wᵀ
    K = 64
    v = np.where(RNG.random(K) < 0.5, -1.0, 1.0)
    u = np.array([0.5, -0.25, 0.125, 1.0])
    w = np.array([2.0, -1.0, 0.75])
    a = _bits(F16, np.outer(u, v))
    b = _bits(F16, np.outer(w, v))
    c, s, _ = orc.gemm(a, b, K, F16, F32)
    assert np.array_equal(s, K * np.outer(u, w))


def pin_small_integer_exact():
    for dtype in (F16, BF16):
        M, N, K = 13, 17, 70
        a = si.make_matrix(M, K, dtype, "small_int", 1)
        b = si.make_matrix(N, K, dtype, "small_int", 2)
        with np.errstate(invalid="ignore"):  # a planted decoding mistake may give NaN; the pin then fails
            ai = orc.decode(dtype, a).astype(np.int64)
            bi = orc.decode(dtype, b).astype(np.int64)
        c, s, t = orc.gemm(a, b, K, dtype, F32)
        assert np.array_equal(s, (ai @ bi.T).astype(np.float64))
        assert np.array_equal(t, (np.abs(ai) @ np.abs(bi).T).astype(np.float64))
        assert np.array_equal(c, (ai @ bi.T).astype(np.float32))


def pin_padding_ignored_and_sampling():
    M, N, K = 6, 5, 40
    a = si.make_matrix(M, K, F16, "uniform", 11, ld=48, pad_bits=0x7E00)  # NaN padding
    b = si.make_matrix(N, K, F16, "uniform", 12, ld=56, pad_bits=0x7C00)  # +inf padding
    a_t = si.make_matrix(M, K, F16, "uniform", 11)
    b_t = si.make_matrix(N, K, F16, "uniform", 12)
    c1, s1, t1 = orc.gemm(a, b, K, F16, F16)
    c2, s2, t2 = orc.gemm(a_t, b_t, K, F16, F16)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.all(np.isfinite(s1))
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    cs, ss, ts = orc.gemm_sampled(a, b, K, F16, F16, ii.ravel(), jj.ravel())
    assert np.array_equal(cs, c1.ravel()) and np.array_equal(ss, s1.ravel()) and np.array_equal(ts, t1.ravel())
    # thread count does not change the result
    c3, s3, _ = orc.gemm(a, b, K, F16, F16, threads=3)
    assert np.array_equal(c3, c1) and np.array_equal(s3, s1)


def pin_empty_cases():
    a = si.make_matrix(4, 8, F16, "uniform", 1)
    b = si.make_matrix(3, 8, F16, "uniform", 2)
    c, s, t = orc.gemm(a, b, 0, F16, F16)  # K = 0: empty sums
    assert np.all(orc.decode(F16, c) == 0.0) and np.all(s == 0) and np.all(t == 0)
    c, s, t = orc.gemm(a[:0], b, 8, F16, F16)
    assert c.shape == (0, 3)


PINS = [pin_f16_decode_exhaustive, pin_f16_encode_vs_numpy, pin_bf16_decode_exhaustive, pin_bf16_encode_vs_torch,
        pin_bf16_single_rounding, pin_generic_encoder_vs_c_float_cast, pin_ulp, pin_ones_closed_form,
        pin_identity_and_permutation, pin_rank1, pin_small_integer_exact, pin_padding_ignored_and_sampling,
        pin_empty_cases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()


# ----------------------------------------------------------------------------- acceptance rule

def test_compare_rule():
    ref = orc.encode(F16, np.array([1.0, 2.0, -3.0, 1000.0]))
    t = np.array([1.0, 2.0, 3.0, 1000.0])
    rep = orc.compare(ref, ref, t, F16, rel=2e-3)
    assert rep["ok"] and rep["max_ratio"] == 0.0
    # one ulp off everywhere: accepted by the ulp term alone
    up = orc.encode(F16, orc.decode(F16, ref) + orc.ulp(F16, orc.decode(F16, ref)))
    assert orc.compare(up, ref, np.zeros(4), F16, rel=2e-3)["ok"]
    # two ulps off with T = 0: rejected
    up2 = orc.encode(F16, orc.decode(F16, ref) + 2 * orc.ulp(F16, orc.decode(F16, ref)))
    rep = orc.compare(up2, ref, np.zeros(4), F16, rel=2e-3)
    assert not rep["ok"] and rep["n_fail"] == 4
    # error within rel*T is accepted, just beyond it is not
    x = np.array([0.5], np.float32)
    ok = np.array([0.5 + 2e-3 * 10 + 2.0 ** -25], np.float32)
    assert orc.compare(ok, x, np.array([10.0]), F32, rel=2e-3)["ok"]
    bad = np.array([0.5 + 2e-3 * 10 + 1e-4], np.float32)
    assert not orc.compare(bad, x, np.array([10.0]), F32, rel=2e-3)["ok"]
    # non-finite output where the reference is finite fails; matching infinities pass
    nan = np.array([np.nan], np.float32)
    assert not orc.compare(nan, x, np.array([1.0]), F32, rel=2e-3)["ok"]
    inf = np.array([np.inf], np.float32)
    assert orc.compare(inf, inf, np.array([1.0]), F32, rel=2e-3)["ok"]
    assert not orc.compare(-inf, inf, np.array([1.0]), F32, rel=2e-3)["ok"]


# ----------------------------------------------------------------------------- planted mistakes

MUTATIONS = {
    "dropped_last_term": ("for (int64_t k = 0; k < j->K; ++k) {\n        s +=",
                          "for (int64_t k = 0; k + 1 < j->K; ++k) {\n        s +="),
    "wrong_sign": ("s += arow[k] * brow[k];", "s -= arow[k] * brow[k];"),
    # A read as if it were stored transposed, wherever that stays inside the buffer
    "transposed_operand": ("arow[k] = oracle_decode(j->in_dtype, j->A[i * j->lda + k]);",
                           "arow[k] = oracle_decode(j->in_dtype, j->A[(k < j->M && i < j->K) ? k * j->lda + i"
                           " : i * j->lda + k]);"),
    "wrong_a_index": ("arow[k] = oracle_decode(j->in_dtype, j->A[i * j->lda + k]);",
                      "arow[k] = oracle_decode(j->in_dtype, j->A[i * j->K + k]);"),
    "abs_sum_not_abs": ("t += fabs(arow[k]) * fabs(brow[k]);", "t += arow[k] * brow[k];"),
    "f16_round_truncates": ("double r = rint(ldexp(a, fbits - e));", "double r = floor(ldexp(a, fbits - e));"),
    "f16_subnormal_decode": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "double_rounding_bf16": ("uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_generic(x, 8, -126, 127, 8); }",
                             "uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_generic((double)(float)x, 8, -126, 127, 8); }"),
    "ulp_off_by_one": ("return ldexp(1.0, e - p + 1);", "return ldexp(1.0, e - p + 2);"),
}


def _build_mutant(src_text, tmpdir, name):
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src_text)
    lib = os.path.join(tmpdir, f"lib{name}.so")
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-pthread", path, "-o", lib, "-lm"], check=True,
                   capture_output=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    src = open(os.path.join(os.path.dirname(orc.__file__), "gemm_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    tmpdir = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        lib_path = _build_mutant(src.replace(old, new), tmpdir, name)
        monkeypatch.setattr(orc, "LIB_PATH", lib_path)
        monkeypatch.setattr(orc, "_lib", None)
        failed = []
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"no pin caught the planted mistake {name}"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
