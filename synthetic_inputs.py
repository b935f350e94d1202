"""Seeded synthetic operands for C = A·Bᵀ, shared by the parity tests, smoke() and bench.py.

This module only makes input bits. It holds none of the product's arithmetic: no dot
products, no accumulation, no output rounding. Both the CPU oracle and the HIP path
receive exactly the bits produced here.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used in counter form: element e of a matrix drawn with seed s
takes the e-th output of a SplitMix64 stream seeded with s, i.e.
``mix64(s + (e + 1) * GOLDEN)``.  Distributions (all computed in float64):

* ``uniform``: ``(h >> 40) * 2**-23 - 1``, i.e. 24-bit uniform on [-1, 1).
* ``normal_scaled``: Box–Muller on the outputs of counters 2e and 2e+1, divided by
  sqrt(K) (the "N(0,1)/sqrt(K)" workload of the 8192³ bf16 headline case).
* ``small_int``: integers in [-3, 3] (``(h >> 32) % 7 - 3``); with K·9 < 2**24 every
  fp32 partial sum of such operands is exact, whatever the summation order.

Each float64 value is then rounded once, to nearest-even, to fp16 or bf16 and returned as
raw 16-bit patterns (``numpy.uint16``).  fp16 uses numpy's float64→float16 conversion;
bf16 rounds the float64 significand to 8 bits in integer arithmetic and keeps the top
half of the (then exact) float32 pattern.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

F16, BF16, F32 = 0, 1, 2
DTYPE_NAMES = {F16: "f16", BF16: "bf16", F32: "f32"}
_CHUNK = 1 << 22


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def splitmix64_stream(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream seeded with ``seed``."""
    e = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + e * GOLDEN
    return mix64(state)


def _values(kind: str, seed: int, start: int, count: int, k: int) -> np.ndarray:
    if kind == "uniform":
        h = splitmix64_stream(seed, start, count)
        return (h >> np.uint64(40)).astype(np.float64) * 2.0 ** -23 - 1.0
    if kind == "normal_scaled":
        h = splitmix64_stream(seed, 2 * start, 2 * count)
        u1 = ((h[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
        u2 = (h[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
        return z / np.sqrt(float(k))
    if kind == "small_int":
        h = splitmix64_stream(seed, start, count)
        return ((h >> np.uint64(32)) % np.uint64(7)).astype(np.float64) - 3.0
    if kind == "ones":
        return np.ones(count, dtype=np.float64)
    raise ValueError(f"unknown distribution {kind!r}")


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to nearest-even fp16; return the bit patterns."""
    return x.astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to nearest-even bf16 (8 significant bits); return bit patterns.

    Valid for zero and for magnitudes in bf16's normal range, which is all the
    distributions above produce; anything else raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.abs(x)
    bad = (a != 0) & ((a < 2.0 ** -126) | ~np.isfinite(a) | (a >= 2.0 ** 127))
    if np.any(bad):
        raise ValueError("to_bf16_bits: value outside bf16's normal range")
    u = x.view(np.uint64).copy()
    drop = np.uint64(45)  # float64 keeps 53 significant bits, bf16 keeps 8
    lsb = (u >> drop) & np.uint64(1)
    u += (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb
    u &= ~((np.uint64(1) << drop) - np.uint64(1))
    f32 = u.view(np.float64).astype(np.float32)  # exact: 8 significant bits, in range
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def make_matrix(rows: int, cols: int, dtype: int, kind: str, seed: int,
                k_for_scale: int | None = None, ld: int | None = None,
                pad_bits: int = 0x7E00) -> np.ndarray:
    """A [rows, ld] uint16 matrix of fp16/bf16 bits; columns >= cols hold ``pad_bits``.

    Element (r, c) with c < cols is element ``r*cols + c`` of the seeded stream, so the
    values do not depend on ``ld``.  ``pad_bits`` defaults to a quiet NaN so that a kernel
    reading the padding of a row shows up in the results.
    """
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    k = cols if k_for_scale is None else k_for_scale
    out = np.full((rows, ld), pad_bits, dtype=np.uint16)
    flat_n = rows * cols
    enc = to_f16_bits if dtype == F16 else to_bf16_bits
    if dtype not in (F16, BF16):
        raise ValueError("inputs are fp16 or bf16")
    flat = out.reshape(-1)
    for s in range(0, flat_n, _CHUNK):
        n = min(_CHUNK, flat_n - s)
        bits = enc(_values(kind, seed, s, n, k))
        if ld == cols:
            flat[s:s + n] = bits
        else:  # scatter the flat chunk into padded rows
            idx = np.arange(s, s + n)
            out[idx // cols, idx % cols] = bits
    return out


def seeds_for(config_index: int, shape_index: int = 0) -> tuple[int, int]:
    """(seed_A, seed_B) for a workload: 0x5EED0000 + 16·config + 2·shape, and that + 1."""
    base = 0x5EED0000 + 16 * config_index + 2 * shape_index
    return base, base + 1


# The five workloads of the headline benchmark table: C = A·Bᵀ with A[M,K], B[N,K] K-major.
WORKLOADS = {
    "c1_256_f16_f32": dict(index=1, shapes=[(256, 256, 256)], in_dtype=F16, out_dtype=F32, dist="uniform"),
    "c2_4096_f16_f16": dict(index=2, shapes=[(4096, 4096, 4096)], in_dtype=F16, out_dtype=F16, dist="uniform"),
    "c3_8192_bf16_bf16": dict(index=3, shapes=[(8192, 8192, 8192)], in_dtype=BF16, out_dtype=BF16,
                              dist="normal_scaled"),
    "c4_16384x16384x1024_bf16": dict(index=4, shapes=[(16384, 16384, 1024)], in_dtype=BF16, out_dtype=BF16,
                                     dist="uniform"),
    "c5_skinny_ragged_f16": dict(index=5, shapes=[(32, 8192, 8192), (4093, 5119, 3071), (8192, 1024, 28672)],
                                 in_dtype=F16, out_dtype=F16, dist="uniform"),
}


def workload_operands(name: str, shape_index: int = 0):
    """(M, N, K, A_bits[M,K], B_bits[N,K], in_dtype, out_dtype) for a named workload."""
    w = WORKLOADS[name]
    m, n, k = w["shapes"][shape_index]
    sa, sb = seeds_for(w["index"], shape_index)
    a = make_matrix(m, k, w["in_dtype"], w["dist"], sa, k_for_scale=k)
    b = make_matrix(n, k, w["in_dtype"], w["dist"], sb, k_for_scale=k)
    return m, n, k, a, b, w["in_dtype"], w["out_dtype"]
