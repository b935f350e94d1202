"""CPU tests of the C-ABI library's host side: exported symbols, argument checking, configuration
choice, the tile scheduler, the LDS swizzle, stage-byte accounting and the ring protocol.

No test here launches GPU work; the scheduler and swizzle checks call host-only entry points
that run the very functions the kernels use.
"""
import json
import math
import os
import re

import pytest

import software_pipelined_tiled_amd as spt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "page_worked_examples.json")))
F16, BF16, F32 = spt.GEMM_F16, spt.GEMM_BF16, spt.GEMM_F32
OK, INVALID, UNSUPPORTED = 0, -1, -2


def header_functions():
    text = open(os.path.join(ROOT, "include", "gemm.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|gemm_status_t|int64_t|int)\s+(gemm_\w+)\s*\(", text, re.M)))


def test_library_exports_every_header_symbol():
    lib = spt.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gemm.h but not exported"
    assert sorted(spt.EXPORTS) == names


def test_status_strings():
    assert spt.status_string(0) == "GEMM_OK"
    assert spt.status_string(-1) == "GEMM_ERR_INVALID"
    assert spt.status_string(-2) == "GEMM_ERR_UNSUPPORTED"
    assert spt.status_string(-3) == "GEMM_ERR_HIP"
    assert spt.status_string(-4) == "GEMM_ERR_NOMEM"
    assert spt.status_string(7) == "GEMM_ERR_UNKNOWN"


@pytest.mark.parametrize("args,status", [
    ((-1, 8, 8, F16, F16, F16, 8, 8, 8), INVALID),
    ((8, -1, 8, F16, F16, F16, 8, 8, 8), INVALID),
    ((8, 8, -1, F16, F16, F16, 8, 8, 8), INVALID),
    ((8, 8, 16, F16, F16, F16, 8, 16, 8), INVALID),       # lda < K
    ((8, 8, 16, F16, F16, F16, 16, 8, 8), INVALID),       # ldb < K
    ((8, 32, 16, F16, F16, F16, 16, 16, 8), INVALID),     # ldc < N
    ((8, 8, 8, F16, BF16, F16, 8, 8, 8), UNSUPPORTED),    # mixed input types
    ((8, 8, 8, F32, F32, F32, 8, 8, 8), UNSUPPORTED),     # fp32 inputs
    ((8, 8, 8, F16, F16, 9, 8, 8, 8), UNSUPPORTED),       # unknown output type
    ((2 ** 31, 8, 8, F16, F16, F16, 8, 8, 8), INVALID),   # size beyond int32
    ((8, 8, 8, F16, F16, F16, 2 ** 31, 8, 8), UNSUPPORTED),
    ((8, 8, 8, F16, F16, F16, 8, 8, 8), OK),
    ((0, 0, 0, F16, F16, F16, 1, 1, 1), OK),              # empty problem
    ((0, 5, 64, F16, F16, F16, 64, 64, 5), OK),           # no output rows, K > 0 (no split of zero tiles)
    ((5, 0, 64, F16, F16, F16, 64, 64, 1), OK),           # no output columns
    ((0, 0, 64, BF16, BF16, F32, 64, 64, 1), OK),
    ((0, 300, 63, F16, F16, F16, 63, 63, 300), OK),       # staged path (K not a multiple of 8)
    ((7, 0, 4096, F16, F16, F16, 4100, 4100, 1), OK),     # staged path through ld
])
def test_argument_checks(args, status):
    assert spt.gemm_select_config_status(*args) == status


def test_plan_create_without_gpu_or_null_out_is_an_error():
    lib = spt.lib()
    assert lib.gemm_plan_create(None, 8, 8, 8, F16, F16, F16, 8, 8, 8, None) == INVALID
    assert lib.gemm_run(None, None, None, None, None) == INVALID
    assert lib.gemm_plan_destroy(None) == OK
    assert lib.gemm_plan_describe(None, None) == INVALID


WORKLOAD_SHAPES = {
    "c1": (256, 256, 256, F16, F32),
    "c2": (4096, 4096, 4096, F16, F16),
    "c3": (8192, 8192, 8192, BF16, BF16),
    "c4": (16384, 16384, 1024, BF16, BF16),
    "c5a": (32, 8192, 8192, F16, F16),
    "c5b": (4093, 5119, 3071, F16, F16),
    "c5c": (8192, 1024, 28672, F16, F16),
}


def ring_bytes(c):
    """LDS of a configuration's ring: S stages of an A and a B K-tile, or, for the split ring (bk
    64, five slots, square tile), five operand slots of one K-tile each."""
    if c["load_path"] != spt.GEMM_LOAD_REG and c["bk"] == 64 and c["stages"] == 5 and c["bm"] == c["bn"]:
        return 5 * c["bm"] * c["bk"] * 2
    return c["stages"] * (c["bm"] + c["bn"]) * c["bk"] * 2


@pytest.mark.parametrize("name", sorted(WORKLOAD_SHAPES))
def test_config_choice(name):
    M, N, K, i, o = WORKLOAD_SHAPES[name]
    c = spt.gemm_select_config(M, N, K, i, i, o, K, K, N, 256, 160 * 1024)
    assert c["lds_bytes"] == ring_bytes(c) <= 160 * 1024
    tiles = math.ceil(M / c["bm"]) * math.ceil(N / c["bn"])
    units = tiles * c["splits"]
    assert 1 <= c["grid"] <= min(units, 512)
    if K % 8 == 0:
        assert c["load_path"] == spt.GEMM_LOAD_DMA
    else:
        # lda = 3071: rows are only 2-byte aligned, so the operands are first copied into rows of 3072
        assert c["load_path"] == spt.GEMM_LOAD_STAGED
    kt = math.ceil(math.ceil(K / 8) * 8 / c["bk"])
    if c["splits"] > 1:
        per = math.ceil(kt / c["splits"])
        assert per >= 8 and (c["splits"] - 1) * per < kt  # every K range non-empty, none tiny
        assert c["splits"] * M * math.ceil(N / 8) * 8 * 4 <= 1 << 30
    if name in ("c2", "c3", "c4"):
        # the two-wave-group kernel with the split ring, whole K per tile
        assert (c["bm"], c["bn"], c["bk"], c["stages"], c["waves"]) == (256, 256, 64, 5, 8) and tiles >= 256
        assert c["lds_bytes"] == 160 * 1024 and c["splits"] == 1
    if name == "c5c":
        assert units >= 256 and c["splits"] > 1  # too few tiles for 256 CUs: K is split to fill them
    if name == "c5a":
        # M = 32: a larger tile would be mostly padding. The time is B streaming in at the HBM rate;
        # 256 workgroups of 32x32 tiles with 128-deep K-tiles stream it (one per 32 columns), so K
        # stays whole and no partial planes are written and reduced
        # B (128 MiB, each tile read by one workgroup) streams with the non-temporal hint through the
        # 8-deep ring
        assert (c["bm"], c["bn"], c["bk"], c["stages"], c["waves"]) == (32, 32, 128, 8, 2) and c["splits"] == 1
        assert c["grid"] == 256 and c["stream"] == 2
    else:
        assert c["stream"] == 0


@pytest.mark.parametrize("M,N,K,tile,stream", [
    (32, 8192, 8192, (32, 32, 128, 8, 2), 2),     # B, 128 MiB, read once: streamed
    (8192, 32, 8192, (32, 32, 128, 8, 2), 1),     # the transpose: A streamed
    (17, 16384, 4096, (32, 32, 128, 8, 2), 2),    # a ragged single tile row, B exactly 128 MiB
    (32, 2048, 8192, (32, 32, 128, 4, 2), 0),     # B of 32 MiB: below the 64 MiB floor, no hint
    (64, 8192, 8192, None, 0),                    # two tile rows of 32 share B: no hint
    (32, 8192, 8191, (32, 32, 128, 8, 2), 2),     # K odd: the staged copy of B is streamed
])
def test_stream_hint_rule(M, N, K, tile, stream):
    c = spt.gemm_select_config(M, N, K, F16, F16, F16, K, K, N, 256, 160 * 1024)
    if tile is not None:
        assert (c["bm"], c["bn"], c["bk"], c["stages"], c["waves"]) == tile
    assert c["stream"] == stream
    assert c["lds_bytes"] == ring_bytes(c)
    if stream == 2:
        assert M <= c["bm"] and 2 * N * K >= 64 << 20
    if stream == 1:
        assert N <= c["bn"] and 2 * M * K >= 64 << 20


def test_staging_needs_each_source_under_2gib():
    # K = 7 rules out the DMA path. The staging copy reaches a source operand through 32-bit byte
    # offsets: 2000 rows of lda = 600000 elements span 2.4 GB, so that plan takes the register path;
    # 1000 rows (1.2 GB) stage as usual
    c = spt.gemm_select_config(2000, 64, 7, F16, F16, F16, 600000, 7, 64, 256, 160 * 1024)
    assert c["load_path"] == spt.GEMM_LOAD_REG
    c = spt.gemm_select_config(1000, 64, 7, F16, F16, F16, 600000, 7, 64, 256, 160 * 1024)
    assert c["load_path"] == spt.GEMM_LOAD_STAGED
    c = spt.gemm_select_config(64, 2000, 7, F16, F16, F16, 7, 600000, 2000, 256, 160 * 1024)
    assert c["load_path"] == spt.GEMM_LOAD_REG


def test_two_part_choice():
    # 4093 x 5119 (K staged to 3072): 320 tiles of 256x256 for 256 workgroups, a second round a
    # quarter full. The plan cuts the columns at 4096 (16 x 16 tiles: one full round of the
    # two-wave-group kernel) and plans the last 1023 columns on their own.
    p = spt.gemm_select_parts(4093, 5119, 3071, F16, F16, F16, 3071, 3071, 5119)
    assert p["dim"] == 1 and p["at"] == 4096
    f, s = p["first"], p["second"]
    assert (f["bm"], f["bn"], f["waves"]) == (256, 256, 8) and math.ceil(4093 / 256) * (4096 // 256) == 256
    assert s["bm"] * s["bn"] < 256 * 256  # the rest runs on smaller tiles
    # shapes that fill whole rounds, or have fewer tiles than workgroups, stay in one part
    for M, N, K in ((8192, 8192, 8192), (4096, 4096, 4096), (16384, 16384, 1024), (32, 8192, 8192),
                    (8192, 1024, 28672), (256, 256, 256)):
        assert spt.gemm_select_parts(M, N, K, BF16, BF16, BF16, K, K, N)["dim"] == -1


@pytest.mark.parametrize("M,N,K", [(4093, 5119, 3072), (5000, 3000, 2048), (3000, 7000, 4096), (4096, 5119, 1024),
                                   (6000, 2100, 8192), (300, 90000, 512)])
def test_two_part_cut_covers_the_output(M, N, K):
    p = spt.gemm_select_parts(M, N, K, F16, F16, F16, K, K, N)
    if p["dim"] < 0:
        return
    f, s, at = p["first"], p["second"], p["at"]
    full = N if p["dim"] == 1 else M
    assert 0 < at < full
    # part 0 ends on a tile edge and runs whole rounds of its tiles (at most one tile line short)
    assert at % (f["bn"] if p["dim"] == 1 else f["bm"]) == 0
    t0 = (math.ceil(M / f["bm"]) * (at // f["bn"]) if p["dim"] == 1 else (at // f["bm"]) * math.ceil(N / f["bn"]))
    g0 = 256 * (1 if f["bm"] * f["bn"] >= 128 * 128 else 2)
    line = math.ceil(M / f["bm"]) if p["dim"] == 1 else math.ceil(N / f["bn"])
    assert t0 % g0 == 0 or g0 - t0 % g0 < line
    assert s["grid"] >= 1 and f["grid"] >= 1


def test_split_choice_small_k_and_limits():
    # K too short to split (fewer than 16 K-tiles): one range per tile
    c = spt.gemm_select_config(64, 64, 512, F16, F16, F16, 512, 512, 64, 256, 160 * 1024)
    assert c["splits"] == 1
    # K = 0: nothing to split
    c = spt.gemm_select_config(64, 64, 0, F16, F16, F16, 8, 8, 64, 256, 160 * 1024)
    assert c["splits"] == 1
    # enough output tiles: no split even with a long K
    c = spt.gemm_select_config(4096, 4096, 65536, BF16, BF16, BF16, 65536, 65536, 4096, 256, 160 * 1024)
    assert c["splits"] == 1
    # a large M*N with few tiles per device slot: the partial planes stay under 1 GiB
    c = spt.gemm_select_config(2048, 2048, 1 << 20, BF16, BF16, F32, 1 << 20, 1 << 20, 2048, 256, 160 * 1024)
    assert c["splits"] * 2048 * 2048 * 4 <= 1 << 30


GOOD_OVERRIDE = dict(bm=128, bn=128, bk=64, stages=4, waves=4, mfma=16, persistent=1, group_m=8, load_path=1,
                     grid=0, lds_bytes=0, splits=1)


@pytest.mark.parametrize("shape,change,status", [
    ((256, 256, 256), dict(bm=96), INVALID),                                  # no such kernel
    ((256, 256, 256), dict(stages=5), INVALID),                               # no 128x128 split ring
    ((256, 256, 256), dict(mfma=32), INVALID),                                # 32x32x16 only in the two-group kernel
    ((256, 256, 256), dict(mfma=8), INVALID),
    ((256, 256, 256), dict(load_path=7), INVALID),
    ((256, 256, 256), dict(bm=256, bn=256, stages=3), INVALID),               # no 4-wave 256x256 three-stage kernel
    ((256, 256, 256), dict(splits=-1), INVALID),
    ((256, 256, 256), dict(splits=17), INVALID),
    ((256, 256, 256), dict(load_path=2, stages=2, splits=2), INVALID),        # register path does not split K
    ((256, 256, 256), dict(persistent=3), INVALID),
    ((256, 256, 256), dict(group_m=-1), INVALID),
    ((256, 256, 100), dict(), INVALID),                                       # DMA forced with K % 8 != 0
    ((256, 256, 256), dict(bm=256, bn=256, stages=5, waves=8, persistent=2), UNSUPPORTED),  # no queue in two-group
    ((256, 256, 256), dict(bm=256, bn=256, stages=5, persistent=2), UNSUPPORTED),  # ring leaves no queue slot
    ((16384, 16384, 1024), dict(splits=2), UNSUPPORTED),                      # partial planes above 1 GiB
    ((256, 256, 256), dict(stream=3), INVALID),
    ((256, 256, 256), dict(stream=-1), INVALID),
    ((256, 256, 256), dict(stream=2), UNSUPPORTED),                           # 128x128 has no hinted variant
    ((32, 256, 256), dict(bm=32, bn=32, bk=128, stages=4, waves=2, load_path=2, stream=2), INVALID),  # no REG 32x32
    ((256, 256, 256), dict(load_path=2, stages=2, stream=1), UNSUPPORTED),    # register path: no hint
])
def test_config_override_validation(shape, change, status):
    # every rejected override returns its own status from the host-only selection and from plan
    # creation, which validates an override before it looks for a device
    import ctypes
    M, N, K = shape
    conf = dict(GOOD_OVERRIDE, **change)
    assert spt.gemm_select_config_status(M, N, K, F16, F16, F16, K, K, N, config=conf) == status
    c = spt.GemmConfig.from_dict(conf)
    p = ctypes.c_void_p()
    assert spt.lib().gemm_plan_create(ctypes.byref(p), M, N, K, F16, F16, F16, K, K, N, ctypes.byref(c)) == status
    assert not p.value


def test_config_override_accepted_and_reported():
    # a valid override is what the plan launches; the grid comes from the device's CU count
    c = spt.gemm_select_config(1000, 700, 512, BF16, BF16, F32, 512, 512, 700, config=GOOD_OVERRIDE)
    assert {k: c[k] for k in ("bm", "bn", "bk", "stages", "waves", "load_path", "splits")} == \
        {"bm": 128, "bn": 128, "bk": 64, "stages": 4, "waves": 4, "load_path": 1, "splits": 1}
    assert c["grid"] == min(256, 8 * 6) and c["lds_bytes"] == 4 * 2 * 128 * 64 * 2
    c = spt.gemm_select_config(1000, 700, 512, BF16, BF16, F32, 512, 512, 700, cu_count=32,
                               config=dict(GOOD_OVERRIDE, splits=3))
    assert c["grid"] == 32 and c["splits"] == 3
    # the streaming hint on request, on the 32x32 tiles, for either operand
    for st in (1, 2):
        c = spt.gemm_select_config(4000, 700, 512, F16, F16, F16, 512, 512, 700, config=dict(
            GOOD_OVERRIDE, bm=32, bn=32, bk=128, stages=8, waves=2, stream=st))
        assert c["stream"] == st and (c["bm"], c["stages"]) == (32, 8)
    # the staged path on request, where DMA cannot read the rows directly
    c = spt.gemm_select_config(100, 70, 77, F16, F16, F16, 77, 77, 70, config=dict(GOOD_OVERRIDE, load_path=3))
    assert c["load_path"] == spt.GEMM_LOAD_STAGED
    # a good override gets past validation; without a GPU plan creation then stops at the device query
    import ctypes
    p = ctypes.c_void_p()
    st = spt.lib().gemm_plan_create(ctypes.byref(p), 1000, 700, 512, BF16, BF16, F32, 512, 512, 700,
                                    ctypes.byref(spt.GemmConfig.from_dict(GOOD_OVERRIDE)))
    assert st == OK or st == -3
    if st == OK:
        spt.lib().gemm_plan_destroy(p)


# ------------------------------------------------------------------------------ scheduler

@pytest.mark.parametrize("tiles_m,tiles_n,splits,group_m,grid", [
    (32, 32, 1, 8, 256), (32, 32, 1, 8, 148), (5, 7, 1, 8, 6), (7, 5, 1, 3, 16), (64, 64, 1, 8, 256),
    (1, 1, 1, 8, 1), (33, 17, 1, 8, 256), (4, 64, 1, 8, 256), (32, 4, 1, 8, 128), (8, 8, 1, 1, 64),
    (3, 3, 1, 2, 1000 // 100), (1, 128, 4, 8, 512), (32, 4, 2, 8, 256), (5, 7, 3, 8, 64), (1, 1, 16, 8, 7)])
def test_schedule_covers_every_unit_once(tiles_m, tiles_n, splits, group_m, grid):
    seen = {}
    per_worker = [0] * grid
    T = tiles_m * tiles_n * splits
    rounds = math.ceil(T / grid)
    for wg in range(grid):
        for r in range(rounds + 1):
            t = spt.gemm_schedule_tile(tiles_m, tiles_n, splits, group_m, grid, wg, r)
            if t is None:
                continue
            assert 0 <= t[0] < tiles_m and 0 <= t[1] < tiles_n and 0 <= t[2] < splits
            assert t not in seen, f"unit {t} assigned twice"
            seen[t] = (wg, r)
            per_worker[wg] += 1
    assert len(seen) == T
    assert max(per_worker) == math.ceil(T / grid)


def test_schedule_split_ranges_run_range_by_range():
    # 8192x1024 at 256x256 with K in two ranges (128 tiles, 256 workgroups): the first round holds
    # every tile once per range, and the workgroups of one XCD share one range
    for x in range(8):
        units = [spt.gemm_schedule_tile(32, 4, 2, 8, 256, wg, 0) for wg in range(x, 256, 8)]
        assert len({u[2] for u in units}) == 1
    first = [spt.gemm_schedule_tile(32, 4, 2, 8, 256, wg, 0) for wg in range(256)]
    assert sorted(first) == sorted((m, n, s) for m in range(32) for n in range(4) for s in range(2))


def test_schedule_page_example_tiles_per_worker():
    g = GOLDEN["persistent_tiles"]
    tm, tn = g["M"] // g["tile"], g["N"] // g["tile"]
    assert tm * tn == g["tiles"]
    counts = [sum(1 for r in range(10) if spt.gemm_schedule_tile(tm, tn, 1, 8, g["workers"], wg, r) is not None)
              for wg in range(g["workers"])]
    assert sum(counts) == g["tiles"]
    assert max(counts) == g["tiles_per_worker_ceil"]


def test_schedule_keeps_each_xcd_on_a_compact_block():
    # 8192^3 at 256x256: 32x32 tiles, 256 workgroups; workgroup w runs on XCD w % 8.
    for r in range(4):
        for x in range(8):
            tiles = [spt.gemm_schedule_tile(32, 32, 1, 8, 256, wg, r) for wg in range(x, 256, 8)]
            rows = {t[0] for t in tiles}
            cols = {t[1] for t in tiles}
            assert len(tiles) == 32 and len(rows) * len(cols) == 32 and len(rows) <= 8 and len(cols) <= 4


def test_schedule_invalid_args():
    with pytest.raises(spt.GemmError):
        spt.gemm_schedule_tile(0, 4, 1, 8, 4, 0, 0)
    with pytest.raises(spt.GemmError):
        spt.gemm_schedule_tile(4, 4, 1, 8, 4, 4, 0)
    with pytest.raises(spt.GemmError):
        spt.gemm_schedule_tile(4, 4, 0, 8, 4, 0, 0)


# ------------------------------------------------------------------------------ LDS layout

@pytest.mark.parametrize("bk", [64, 128])
def test_lds_layout_is_a_bijection(bk):
    rows = 256
    offs = {spt.gemm_lds_chunk_offset(rows, bk, r, c) for r in range(rows) for c in range(bk // 8)}
    assert offs == set(range(0, rows * bk * 2, 16))
    assert spt.gemm_lds_chunk_offset(rows, bk, rows, 0) == -1
    assert spt.gemm_lds_chunk_offset(rows, 96, 0, 0) == -1


def test_lds_page_bank_example():
    g = GOLDEN["bank_sectors"]
    # a 16 x 128 fp16 slice (256-byte rows) staged as two 128-byte groups (depth 128 = 2 groups);
    # 32 banks x 4 bytes: a 16-byte chunk at byte X uses bank sector (X // 16) % 8
    for col in range(16):
        sectors = {(spt.gemm_lds_chunk_offset(16, 128, row, col) // 16) % 8 for row in range(g["rows"])}
        assert len(sectors) == g["grouped_distinct"]
    # the ungrouped comparison printed on the page: sector = local_col XOR ((2*row + col//8) % 8)
    for col in range(16):
        sectors = {(col % 8) ^ ((2 * row + col // 8) % 8) for row in range(g["rows"])}
        assert len(sectors) == g["ungrouped_distinct"]


def test_lds_swizzle_spreads_every_eight_row_column():
    # the property the pages state for the 128-byte swizzle: the same logical 16-byte chunk of
    # eight consecutive rows sits in eight different physical chunk positions (bank sectors)
    for bk in (64, 128):
        for base in range(0, 256, 8):
            for c in range(bk // 8):
                pos = {(spt.gemm_lds_chunk_offset(256, bk, base + i, c) % 128) // 16 for i in range(8)}
                assert len(pos) == 8


# ------------------------------------------------------------------------------ stage bytes

DMA_TABLE = [(256, 256, 2), (256, 256, 1), (256, 128, 3), (256, 128, 2), (256, 128, 1), (128, 128, 4),
             (128, 128, 3), (128, 128, 2), (128, 128, 1), (64, 64, 4), (64, 64, 2)]
# (bm, bn, bk, stages, waves) of the configurations with their own ring shape
RING_TABLE = [(256, 256, 64, 5, 4), (256, 256, 32, 4, 4), (256, 256, 64, 5, 8), (256, 256, 64, 2, 8),
              (64, 64, 128, 4, 4), (32, 32, 128, 4, 2), (32, 32, 128, 8, 2)]


def stage_bytes(bm, bn, bk, elem=2):
    return (bm * bk + bn * bk) * elem


def test_stage_bytes_page_example():
    g = GOLDEN["stage_bytes"]
    # a 16x64 fp16 A tile and a 16x64 fp16 B tile are 2048 bytes each
    assert 16 * 64 * 2 == g["a_bytes"] and stage_bytes(16, 16, 64) == g["total"]


@pytest.mark.parametrize("bm,bn,s", DMA_TABLE)
def test_stage_accounting_of_every_dma_config(bm, bn, s):
    waves, bk = 4, 64
    total = stage_bytes(bm, bn, bk)
    # every wave issues the same number of 1 KiB direct-to-LDS loads per stage
    assert total % (1024 * waves) == 0
    lw = total // (1024 * waves)
    # vmcnt thresholds used by the ring: lw * (S-2) in steady state, up to lw * (S-1) after the prologue
    assert lw * max(s - 1, 1) < 64
    assert s * total <= 160 * 1024


@pytest.mark.parametrize("bm,bn,bk,s,waves", RING_TABLE)
def test_stage_accounting_of_ring_configs(bm, bn, bk, s, waves):
    cfg = dict(bm=bm, bn=bn, bk=bk, stages=s, waves=waves, load_path=spt.GEMM_LOAD_DMA)
    assert ring_bytes(cfg) <= 160 * 1024
    if waves == 8:
        # one group of four waves loads an operand tile: 1 KiB per instruction
        la = bm * bk * 2 // (1024 * 4)
        assert la == 8 and (bm * bk * 2) % (1024 * 4) == 0
        assert la * 2 < 64  # the largest threshold: a stage, or an operand tile plus one in flight
    elif s == 5 and bk == 64:
        la, lb = bm * bk * 2 // (1024 * waves), bn * bk * 2 // (1024 * waves)
        assert 2 * la + lb < 64  # prologue threshold of the split ring
    else:
        lw = stage_bytes(bm, bn, bk) // (1024 * waves)
        assert lw * (s - 1) < 64


# ------------------------------------------------------------------------------ ring protocol replay
#
# The replays below take every wait threshold and refill count from gemm_pipeline_protocol, which
# returns the constants the kernels are compiled with (both read the same constexpr function), so a
# threshold that would let a wave read a K-tile before it landed, or refill a slot another wave is
# still reading, fails here without a GPU.

# (bm, bn, bk, stages, waves) of every DMA mainloop kernel
PLAIN_KERNELS = [(256, 256, 64, 2, 4), (256, 256, 32, 4, 4), (256, 256, 64, 1, 4), (256, 128, 64, 3, 4),
                 (256, 128, 64, 2, 4), (256, 128, 64, 1, 4), (128, 128, 64, 4, 4), (128, 128, 64, 3, 4),
                 (128, 128, 64, 2, 4), (128, 128, 64, 1, 4), (64, 64, 64, 4, 4), (64, 64, 128, 4, 4),
                 (64, 64, 64, 2, 4), (32, 32, 128, 4, 2), (32, 32, 128, 8, 2)]
SPLIT_KERNELS = [(256, 256, 64, 5, 4)]
TWO_GROUP_KERNELS = [(256, 256, 64, 5, 8), (256, 256, 64, 2, 8)]


def protocol(cfg):
    p = spt.gemm_pipeline_protocol(*cfg)
    assert p is not None, f"no kernel {cfg}"
    return p


def test_protocol_export_matches_kernel_tables():
    for cfg in PLAIN_KERNELS + SPLIT_KERNELS + TWO_GROUP_KERNELS:
        bm, bn, bk, s, w = cfg
        p = protocol(cfg)
        issuers = 4 if w == 8 else w
        assert p["la"] * issuers * 1024 == bm * bk * 2 and p["lb"] * issuers * 1024 == bn * bk * 2
        assert p["split"] == (1 if (bk, s) == (64, 5) else 0)
        assert max(p["prologue_wait"], p["handover_wait"]) < 64  # the 6-bit vmcnt field
    assert spt.gemm_pipeline_protocol(96, 64, 64, 2, 4) is None


def replay_ring(KT, S, p, wait_slack=0, refill_before_barrier=False):
    """Replay the 4-wave kernel's K-loop for one wave (waves are symmetric; a barrier is a point all
    of them reach). Loads complete in issue order; vmcnt(n) returns once at most n of this wave's
    loads are outstanding. K-tiles past the end are zero-filling dummies (they still write LDS).
    Checks: a K-tile is read only after all its loads landed, and a slot is refilled only after
    every wave finished reading the K-tile it held."""
    LW = p["lw"]
    issued = []          # K-tile of each issued load, in order
    slot_tile = {}       # slot -> K-tile it holds (or is receiving)
    reads_done = set()   # K-tiles every wave has finished reading (lgkmcnt(0), then the barrier)
    state = {"landed_upto": -1}

    def issue(tile, n):
        slot = tile % S
        if slot_tile.get(slot) != tile:
            prev = slot_tile.get(slot)
            assert prev is None or prev in reads_done, f"slot {slot} refilled with K-tile {tile} before K-tile {prev} was read"
            slot_tile[slot] = tile
        issued.extend([tile] * n)

    def wait_vm(n):
        state["landed_upto"] = max(state["landed_upto"], len(issued) - 1 - n)

    def landed(tile):
        idx = [i for i, t in enumerate(issued) if t == tile]
        return len(idx) == LW and max(idx) <= state["landed_upto"] and slot_tile[tile % S] == tile

    for t in range(S):  # prologue: the first S K-tiles (dummies past the end included)
        issue(t, LW)
    wait_vm(p["prologue_wait"] + wait_slack)
    assert landed(0), "K-tile 0 read before it landed"
    for k in range(KT):
        if k >= 1 and p["refill_later"]:
            issue(k - 1 + S, p["refill_later"])  # k-step 0: the rest of the refill begun at the last hand-over
        if k + 1 == KT:
            reads_done.add(k)
            break
        # hand-over: lgkmcnt(0), vmcnt(handover_wait), barrier, then the refill of K-tile k+S
        if S == 1:
            reads_done.add(k)
            issue(k + 1, LW)
            wait_vm(0)
        else:
            if refill_before_barrier:
                issue(k + S, p["refill_now"])  # planted mistake: the refill before the barrier
            wait_vm(p["handover_wait"] + wait_slack)
            reads_done.add(k)
            issue(k + S, p["refill_now"])
        assert landed(k + 1), f"K-tile {k + 1} read before it landed (KT={KT}, S={S})"


def replay_ring_units(units, KT, S, p, store_credit=0):
    """The 4-wave kernel over `units` work units in a row, as one wave runs them: per unit a prologue,
    the K-loop and 16 epilogue stores, the ring restarting at slot 0 while the previous unit's
    zero-filling dummy K-tiles may still be in flight into the same slots. vmcnt counts loads and
    stores; stores may complete before any load, loads complete in issue order, so every wait is
    replayed with the stores completing first. A slot's new load may be issued while an older load
    into it is in flight only because this wave's loads land in order; the check is that every read
    finds the newest load of its slot landed and that the slot holds the K-tile it reads."""
    LW, NS = p["lw"], 16
    ops = []                 # ("L", unit, tile) or ("S",)
    done = set()
    holds = {}               # slot -> (unit, tile) of its newest load

    def issue(u, tile, n):
        holds[tile % S] = (u, tile)
        ops.extend([("L", u, tile)] * n)

    def wait(n):
        out = [i for i in range(len(ops)) if i not in done]
        for i in [i for i in out if ops[i][0] == "S"] + [i for i in out if ops[i][0] == "L"]:
            if len(ops) - len(done) <= n:
                break
            done.add(i)

    def readable(u, tile):
        idx = [i for i, o in enumerate(ops) if o[0] == "L" and o[1] == u and o[2] == tile]
        return len(idx) == LW and all(i in done for i in idx) and holds[tile % S] == (u, tile)

    for u in range(units):
        for t in range(S):
            issue(u, t, LW)
        wait(p["prologue_wait"] + (store_credit if u else 0))
        assert readable(u, 0), f"unit {u}: K-tile 0 read before it landed"
        for k in range(KT):
            if k >= 1 and p["refill_later"]:
                issue(u, k - 1 + S, p["refill_later"])
            if k + 1 == KT:
                break
            if S == 1:
                issue(u, k + 1, LW)
                wait(0)
            else:
                wait(p["handover_wait"])
                issue(u, k + S, p["refill_now"])
            assert readable(u, k + 1), f"unit {u}: K-tile {k + 1} read before it landed"
        ops.extend([("S",)] * NS)


@pytest.mark.parametrize("cfg", PLAIN_KERNELS)
def test_ring_protocol_replay_over_units_with_stores(cfg):
    p = protocol(cfg)
    S = cfg[3]
    for KT in range(1, 2 * S + 3):
        replay_ring_units(3, KT, S, p)


def test_ring_units_replay_catches_a_wait_that_trusts_store_order():
    p = protocol((128, 128, 64, 4, 4))
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 8):
            replay_ring_units(3, KT, 4, p, store_credit=16)


@pytest.mark.parametrize("cfg", PLAIN_KERNELS)
def test_ring_protocol_replay(cfg):
    p = protocol(cfg)
    S = cfg[3]
    for KT in range(1, 2 * S + 4):
        replay_ring(KT, S, p)


@pytest.mark.parametrize("cfg", [c for c in PLAIN_KERNELS if c[3] >= 2])
def test_ring_replay_catches_planted_mistakes(cfg):
    p = protocol(cfg)
    S = cfg[3]
    # a vmcnt threshold one load too lax lets a wave read a K-tile that has not fully landed
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 2 * S + 4):
            replay_ring(KT, S, p, wait_slack=1)
    # refilling a slot before the barrier overwrites a K-tile other waves may still be reading
    with pytest.raises(AssertionError, match="refilled"):
        for KT in range(1, 2 * S + 4):
            replay_ring(KT, S, p, refill_before_barrier=True)


# The split ring (five operand slots of one K-tile each): K-tile k's A tile is operand tile 2k, its B
# tile 2k+1, and operand tile h sits in slot h mod 5. The prologue loads operand tiles 0 .. 4; at the
# hand-over of K-tile k the wave waits, syncs and loads B(k+2) (refill_now loads) in the hand-over
# k-step; k-step 0 of K-tile k+1 loads A(k+3) (refill_later loads). Tiles past the end are dummies.
def replay_split_ring(KT, p, wait_slack=0, early_b=False):
    LA, LB = p["la"], p["lb"]
    assert (p["refill_now"], p["refill_later"]) == (LB, LA)
    issued = []        # operand tile of each load, in order
    slot_of = {}       # slot -> operand tile it holds
    read = set()       # K-tiles whose fragment reads completed everywhere
    state = {"landed_upto": -1}

    def load(h):
        slot = h % 5
        prev = slot_of.get(slot)
        if prev is not None:
            assert prev // 2 in read, f"slot {slot} refilled with operand tile {h} before K-tile {prev // 2} was read"
        slot_of[slot] = h
        issued.extend([h] * (LA if h % 2 == 0 else LB))

    def wait_vm(n):
        state["landed_upto"] = max(state["landed_upto"], len(issued) - 1 - n)

    def landed(k):
        idx = [i for i, h in enumerate(issued) if h in (2 * k, 2 * k + 1)]
        return (idx and max(idx) <= state["landed_upto"] and slot_of[(2 * k) % 5] == 2 * k
                and slot_of[(2 * k + 1) % 5] == 2 * k + 1)

    for h in range(5):
        load(h)
    wait_vm(p["prologue_wait"] + wait_slack)
    assert landed(0), "K-tile 0 read before it landed"
    for k in range(KT):
        if k >= 1:
            load(2 * (k + 2))                 # A(k+2), k-step 0 of K-tile k
        if k + 1 == KT:
            read.add(k)
            break
        if early_b:
            load(2 * (k + 2) + 1)             # planted mistake: B(k+2) before the hand-over barrier
        wait_vm(p["handover_wait"] + wait_slack)
        read.add(k)                           # hand-over barrier: every wave's reads of K-tile k are done
        assert landed(k + 1), f"K-tile {k + 1} read before it landed (KT={KT})"
        if not early_b:
            load(2 * (k + 2) + 1)             # B(k+2), hand-over k-step


@pytest.mark.parametrize("cfg", SPLIT_KERNELS)
def test_split_ring_replay(cfg):
    p = protocol(cfg)
    for KT in range(1, 12):
        replay_split_ring(KT, p)
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 12):
            replay_split_ring(KT, p, wait_slack=1)
    with pytest.raises(AssertionError, match="refilled"):
        for KT in range(1, 12):
            replay_split_ring(KT, p, early_b=True)


# The two-wave-group schedule. Phases are separated by workgroup barriers; K-tile u is read by G0 in
# phase 2u and by G1 in phase 2u+1. S = 2: G0 loads K-tile u+1 (both operand tiles) in phase 2u and
# waits vmcnt(0) at the end of phase 2u+1. S = 5 (split): G0 loads B(u+1) in phase 2u and waits
# vmcnt(0) at the end of phase 2u+1; G1 loads A(u+2) in phase 2u+1 and, at the end of that phase,
# waits vmcnt(pp_g1_wait) (vmcnt(0) when it loaded nothing). The prologue (G0) loads A(0), B(0) and,
# for S = 5, A(1), then waits vmcnt(pp_g0_prologue_wait). This replays one work unit; the kernel's
# phase stream continues into the next unit the same way (the cursors then point into it).
def replay_two_groups(KT, S, p, g1_slack=0, g0_late_wait=False, g0_prologue_slack=0):
    LA = p["la"]
    loads = {0: [], 1: []}       # per group: operand tile of each load, in order
    landed = {0: -1, 1: -1}
    slot_of = {}
    read_done = {}               # K-tile -> phase after which both groups finished reading it

    def slot(h):
        return h % 5 if S == 5 else (h // 2) % 2 * 2 + h % 2   # S = 2: stage (k mod 2), A or B half

    def load(g, h, phase):
        sl = slot(h)
        prev = slot_of.get(sl)
        if prev is not None:
            assert read_done.get(prev // 2, 1 << 30) < phase, f"slot {sl} refilled in phase {phase} before K-tile {prev // 2} was read"
        slot_of[sl] = h
        loads[g].extend([h] * LA)

    def wait(g, n):
        landed[g] = max(landed[g], len(loads[g]) - 1 - n)

    def is_landed(h):
        for g in (0, 1):
            idx = [i for i, x in enumerate(loads[g]) if x == h]
            if idx:
                return max(idx) <= landed[g] and slot_of[slot(h)] == h
        return False

    def check_read(u, phase):
        for h in (2 * u, 2 * u + 1):
            assert is_landed(h), f"operand tile {h} read in phase {phase} before it landed (KT={KT}, S={S})"

    load(0, 0, -1)
    load(0, 1, -1)
    if S == 5 and KT > 1:
        load(0, 2, -1)
        wait(0, p["pp_g0_prologue_wait"] + g0_prologue_slack)
    else:
        wait(0, 0)
    for u in range(KT):
        p0, p1 = 2 * u, 2 * u + 1
        # phase 2u: G0 memory (loads, then reads K-tile u); G1 computes K-tile u-1
        if u + 1 < KT:
            if S == 5:
                load(0, 2 * (u + 1) + 1, p0)
            else:
                load(0, 2 * (u + 1), p0)
                load(0, 2 * (u + 1) + 1, p0)
        check_read(u, p0)
        # phase 2u+1: G0 computes K-tile u, then waits; G1 memory (loads, reads K-tile u, waits)
        g1_loaded = False
        if S == 5 and u + 2 < KT:
            load(1, 2 * (u + 2), p1)
            g1_loaded = True
        check_read(u, p1)
        read_done[u] = p1
        if not g0_late_wait:
            wait(0, 0)
        if S == 5:
            wait(1, (p["pp_g1_wait"] if g1_loaded else 0) + g1_slack)


def replay_two_group_stream(units, KT, S, p, store_credit=0):
    """The two-group phase stream over `units` work units of KT K-tiles, run back to back as the
    kernel runs them (loads run ahead into the next unit; no ring reset between units), with each
    finished unit's 16 stores per wave issued where the kernel issues them: G0 after its B loads in
    the first memory phase of the next unit, G1 after its wait in its first memory phase, and both
    after the last unit. vmcnt counts loads and stores, and a store may complete before or after any
    load, so each wait is replayed adversarially: the stores complete first, then the oldest loads,
    until at most n operations are outstanding. store_credit plants a wait that counts the stores as
    if they completed in order (threshold raised by that many)."""
    LA, NS = p["la"], 16
    ops = {0: [], 1: []}          # per group, in issue order: ("L", operand tile) or ("S", None)
    done = {0: set(), 1: set()}   # indices of completed operations
    slot_of, read_done = {}, {}

    def slot(h):
        return h % 5 if S == 5 else (h // 2) % 2 * 2 + h % 2

    def load(g, h, phase):
        prev = slot_of.get(slot(h))
        if prev is not None:
            assert read_done.get(prev // 2, 1 << 30) < phase, f"slot refilled in phase {phase} before K-tile {prev // 2} was read"
        slot_of[slot(h)] = h
        ops[g].extend([("L", h)] * LA)

    def store(g):
        ops[g].extend([("S", None)] * NS)

    def wait(g, n):
        out = [i for i in range(len(ops[g])) if i not in done[g]]
        for i in [i for i in out if ops[g][i][0] == "S"] + [i for i in out if ops[g][i][0] == "L"]:
            if len(ops[g]) - len(done[g]) <= n:
                break
            done[g].add(i)

    def is_landed(h):
        for g in (0, 1):
            idx = [i for i, (k, x) in enumerate(ops[g]) if k == "L" and x == h]
            if idx:
                return all(i in done[g] for i in idx) and slot_of[slot(h)] == h
        return False

    def check_read(u, phase):
        for h in (2 * u, 2 * u + 1):
            assert is_landed(h), f"operand tile {h} read in phase {phase} before it landed"

    G = units * KT
    load(0, 0, -1)
    load(0, 1, -1)
    if S == 5 and G > 1:
        load(0, 2, -1)
        wait(0, p["pp_g0_prologue_wait"])
    else:
        wait(0, 0)
    for u in range(G):
        first = u % KT == 0 and u > 0            # the first K-tile of a unit after the first: epilogue
        p0, p1 = 2 * u, 2 * u + 1
        if u + 1 < G:
            if S == 5:
                load(0, 2 * (u + 1) + 1, p0)
            else:
                load(0, 2 * (u + 1), p0)
                load(0, 2 * (u + 1) + 1, p0)
        if first:
            store(0)
        check_read(u, p0)
        g1_loaded = False
        if S == 5 and u + 2 < G:
            load(1, 2 * (u + 2), p1)
            g1_loaded = True
        if S == 5:
            wait(1, (p["pp_g1_wait"] if g1_loaded else 0) + (store_credit if any(k == "S" for k, _ in ops[1]) else 0))
        if first:
            store(1)
        check_read(u, p1)
        read_done[u] = p1
        wait(0, 0)
    store(0)
    store(1)


@pytest.mark.parametrize("cfg", TWO_GROUP_KERNELS)
def test_two_group_stream_with_stores_replay(cfg):
    p = protocol(cfg)
    for units in (1, 2, 3):
        for KT in (1, 2, 3, 5, 8):
            replay_two_group_stream(units, KT, cfg[3], p)


def test_two_group_stream_replay_catches_a_wait_that_trusts_store_order():
    # a G1 wait that treats the stores issued after A(g+1)'s loads as completing in order (raising its
    # threshold by their count) lets a read of A(g+1) run before it lands
    p5 = protocol((256, 256, 64, 5, 8))
    with pytest.raises(AssertionError, match="before it landed"):
        for units in (2, 3):
            for KT in (2, 3, 5):
                replay_two_group_stream(units, KT, 5, p5, store_credit=16)


@pytest.mark.parametrize("cfg", TWO_GROUP_KERNELS)
def test_two_group_schedule_replay(cfg):
    p = protocol(cfg)
    for KT in range(1, 12):
        replay_two_groups(KT, cfg[3], p)


def test_two_group_replay_catches_planted_mistakes():
    p5 = protocol((256, 256, 64, 5, 8))
    p2 = protocol((256, 256, 64, 2, 8))
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 12):
            replay_two_groups(KT, 5, p5, g1_slack=1)
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 12):
            replay_two_groups(KT, 5, p5, g0_prologue_slack=1)
    with pytest.raises(AssertionError, match="before it landed"):
        for KT in range(1, 12):
            replay_two_groups(KT, 2, p2, g0_late_wait=True)


@pytest.mark.parametrize("M,N,K", [(0, 5, 64), (5, 0, 64), (0, 0, 1), (0, 4096, 8192), (8192, 0, 28672)])
def test_empty_output_plans_on_every_path(M, N, K):
    # M or N = 0 with K > 0 is a no-op; the choice must not divide by the zero tile count on any path
    for lda in (K, K + 1, K + 8):
        for cu, lds in ((256, 160 * 1024), (1, 65536)):
            assert spt.gemm_select_config_status(M, N, K, F16, F16, F16, lda, lda, max(N, 1), cu, lds) == OK
            c = spt.gemm_select_config(M, N, K, F16, F16, F16, lda, lda, max(N, 1), cu, lds)
            assert c["grid"] >= 1 and c["splits"] == 1
