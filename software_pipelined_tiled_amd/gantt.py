"""The two-lane pipeline model of "GEMM II — pipelining with TMA" (Interactive · the pipeline
Gantt): one lane for the load engine, one for the matrix unit, a K-loop of tiles through a ring of
``depth`` slots, with a fixed load time and a fixed MMA time per K-tile.

* ``serial`` (Step 4): load K-tile k, wait for it, run its MMA, wait for that, then load k+1.
* ``prefetch`` (Step 5): the prologue issues the loads of K-tiles 0 .. depth-1; iteration k waits
  for K-tile k, runs its MMA and waits for it (the MMA gates every iteration, as the page stresses),
  then issues the load of K-tile k+depth into the slot k just freed. Loads are a fixed latency and
  may overlap, so at most ``depth`` are in flight.

The page's KPIs are reported: the makespan, the fraction of it the matrix unit is idle, whether the
MMAs run back to back, and the largest number of loads in flight. Reading of the page: its widget
gives the model's inputs (a fixed load and MMA time per tile, the ring depth, the tile count) but
its KPI values did not survive extraction, so the recurrence below is the plain reading of Step 5's
loop structure (issue k+depth after MMA k completes), pinned by closed forms in the tests.

With ``depth`` = 1 the prefetch loop is the serial loop. When a load fits behind depth-1 MMAs
(load <= (depth-1) * mma) only the first load is exposed: makespan = load + k_tiles * mma. Otherwise
the steady-state period per K-tile is (load + mma) / depth.
"""
from __future__ import annotations


def simulate(k_tiles: int, depth: int, load: float, mma: float, mode: str = "prefetch") -> dict:
    if k_tiles < 0 or depth < 1 or load < 0 or mma < 0:
        raise ValueError("k_tiles >= 0, depth >= 1, load >= 0, mma >= 0")
    if mode not in ("serial", "prefetch"):
        raise ValueError("mode is 'serial' or 'prefetch'")
    issue, land, start, end = [], [], [], []
    for k in range(k_tiles):
        if mode == "serial":
            i = end[k - 1] if k else 0.0
        else:
            i = 0.0 if k < depth else end[k - depth]
        issue.append(i)
        land.append(i + load)
        s = max(land[k], end[k - 1] if k else 0.0)
        start.append(s)
        end.append(s + mma)
    makespan = end[-1] if k_tiles else 0.0
    busy = k_tiles * mma
    # loads in flight at each instant a load is issued (a load counts from its issue until it lands)
    in_flight = max((sum(1 for j in range(k_tiles) if issue[j] <= t < land[j]) for t in issue), default=0)
    eps = 1e-12 * max(1.0, makespan)
    return {
        "makespan": makespan,
        "idle": (1.0 - busy / makespan) if makespan > 0 else 0.0,
        "back_to_back": all(start[k] <= end[k - 1] + eps for k in range(1, k_tiles)),
        "max_loads_in_flight": in_flight,
        "mma_start": start,
        "load_issue": issue,
    }


def predict_rounds(k_tiles: int, depth: int, load: float, mma: float, rounds: int) -> float:
    """Time of `rounds` output tiles per workgroup, each a K-loop of `k_tiles` through the ring
    (the ring restarts per tile, as in the page's persistent loop, which resets its phases per tile)."""
    mode = "serial" if depth == 1 else "prefetch"
    return rounds * simulate(k_tiles, depth, load, mma, mode)["makespan"]
