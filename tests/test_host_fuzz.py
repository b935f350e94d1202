"""Host-only entry points on arbitrary arguments (CPU): each returns a status and never traps.

The seeded random sweep runs in a child process (tests/host_fuzz_driver.py), so that a trap ends only
that process and its last printed line names the arguments. The named cases are the inputs that
trapped before: a split choice dividing by a zero tile count, a raster band whose height times the
tile columns overflowed 32 bits, and a two-part search over every round count of a huge grid."""
import ctypes
import os
import subprocess
import sys
import time

import pytest

import software_pipelined_tiled_amd as spt

HERE = os.path.dirname(os.path.abspath(__file__))
F16 = 0


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_random_host_calls_return_a_status(seed):
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_fuzz_driver.py"), str(seed), "1500"],
                       capture_output=True, text=True, timeout=600)
    last = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    assert r.returncode == 0, f"exit {r.returncode}; last call: {last}\n{r.stderr[-2000:]}"
    assert last == "done 1500"


def test_empty_output_with_k_does_not_divide_by_zero():
    assert spt.gemm_select_config_status(0, 0, 1, F16, F16, F16, 1, 1, 1) == 0
    assert spt.gemm_select_config_status(0, 5, 64, F16, F16, F16, 64, 64, 5) == 0


def test_tall_raster_band_is_clamped_to_the_grid():
    lib = spt.lib()
    tm, tn, s = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    # group_m x tiles_n = 2^32: the band is the whole grid, ordered column by column
    assert lib.gemm_schedule_tile(33, 65536, 8, 65536, 4096, 257, 1, ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(s)) == 1
    assert 0 <= tm.value < 33 and 0 <= tn.value < 65536 and 0 <= s.value < 8
    for wg in (0, 1, 4095):
        ref = (ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int())
        got = (ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int())
        assert lib.gemm_schedule_tile(33, 65536, 8, 33, 4096, wg, 3, *map(ctypes.byref, ref)) == 1
        assert lib.gemm_schedule_tile(33, 65536, 8, 1 << 20, 4096, wg, 3, *map(ctypes.byref, got)) == 1
        assert [v.value for v in ref] == [v.value for v in got]
    # an override with a band taller than the grid plans, and runs with the grid's height
    cfg = dict(bm=128, bn=128, bk=64, stages=4, waves=4, mfma=16, persistent=1, group_m=1 << 30, load_path=1, grid=0,
               lds_bytes=0, splits=1, stream=0)
    c = spt.gemm_select_config(1000, 70000, 64, F16, F16, F16, 64, 64, 70000, config=cfg)
    assert c["group_m"] == 8  # ceil(1000 / 128) tile rows


def test_two_part_search_is_bounded_for_huge_grids():
    t0 = time.perf_counter()
    spt.gemm_select_config_status((1 << 31) - 1, 1 << 20, 1 << 20, F16, F16, F16, 1 << 20, 1 << 20, 1 << 20)
    try:
        spt.gemm_select_parts((1 << 31) - 1, 1 << 20, 1 << 20, F16, F16, F16, 1 << 20, 1 << 20, 1 << 20)
    except spt.GemmError:
        pass
    assert time.perf_counter() - t0 < 1.0
