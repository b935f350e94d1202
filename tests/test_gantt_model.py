"""The pipeline Gantt model ("GEMM II — pipelining with TMA", Interactive · the pipeline Gantt)
against closed forms of its two schedules; the page's own KPI values did not survive extraction,
so these are the pins."""
import math

import pytest

from software_pipelined_tiled_amd import gantt


@pytest.mark.parametrize("k,load,mma", [(8, 1.2, 1.0), (1, 3.0, 2.0), (16, 0.5, 1.0), (5, 0.0, 1.0), (7, 2.0, 0.0)])
def test_serial_is_load_plus_mma_per_tile(k, load, mma):
    r = gantt.simulate(k, 1, load, mma, "serial")
    assert math.isclose(r["makespan"], k * (load + mma))
    assert r["max_loads_in_flight"] == (1 if load > 0 else 0)
    # prefetch with a one-slot ring is the same loop
    p = gantt.simulate(k, 1, load, mma, "prefetch")
    assert math.isclose(p["makespan"], r["makespan"])


@pytest.mark.parametrize("depth,load,mma,k", [(2, 1.0, 1.0, 8), (3, 1.9, 1.0, 10), (4, 3.0, 1.0, 12), (2, 0.3, 1.0, 1)])
def test_load_hidden_behind_depth_minus_one_mmas(depth, load, mma, k):
    # load <= (depth-1) * mma: only the first load is exposed and the MMAs run back to back
    r = gantt.simulate(k, depth, load, mma)
    assert math.isclose(r["makespan"], load + k * mma)
    assert r["back_to_back"]
    assert math.isclose(r["idle"], load / (load + k * mma))
    assert r["max_loads_in_flight"] == min(depth, k)


@pytest.mark.parametrize("depth,load,mma", [(2, 1.2, 1.0), (2, 3.0, 1.0), (3, 4.0, 1.0), (4, 7.0, 0.5)])
def test_load_bound_period(depth, load, mma):
    # load > (depth-1) * mma: each slot turns over once per load + mma, so K-tile k + depth starts
    # load + mma after K-tile k; the makespan of K = depth * n tiles follows exactly
    n = 6
    k = depth * n
    r = gantt.simulate(k, depth, load, mma)
    assert not r["back_to_back"]
    starts = r["mma_start"]
    for i in range(depth, k):
        assert math.isclose(starts[i] - starts[i - depth], load + mma)
    assert math.isclose(r["makespan"], load + (n - 1) * (load + mma) + depth * mma)


def test_page_widget_parameters():
    # the widget's defaults: PIPE_DEPTH 2, 8 K-tiles, load:MMA 1.2. Prefetch cuts the makespan from
    # 8 x 2.2 to 9.8 (first load, then the two slots turning over every 2.2)
    s = gantt.simulate(8, 2, 1.2, 1.0, "serial")
    p = gantt.simulate(8, 2, 1.2, 1.0, "prefetch")
    assert math.isclose(s["makespan"], 17.6) and math.isclose(s["idle"], 9.6 / 17.6)
    assert math.isclose(p["makespan"], 9.8) and math.isclose(p["idle"], 1 - 8 / 9.8)
    assert p["max_loads_in_flight"] == 2
    # a third slot hides a 1.2 load completely
    assert gantt.simulate(8, 3, 1.2, 1.0)["back_to_back"]


def test_rejects_bad_arguments():
    for args in ((-1, 2, 1.0, 1.0), (4, 0, 1.0, 1.0), (4, 2, -1.0, 1.0)):
        with pytest.raises(ValueError):
            gantt.simulate(*args)
    with pytest.raises(ValueError):
        gantt.simulate(4, 2, 1.0, 1.0, "other")
    assert gantt.simulate(0, 2, 1.0, 1.0)["makespan"] == 0.0
