"""GPU parity at the workloads' full shapes.

Every call runs on the full state set of the workload (all units and heads,
so the launch configuration is the benchmark's: same grids, same per-call
state size and therefore the same cached / streaming choice for the state
traffic), for fewer steps than the benchmark times.  The float64 oracle then
checks a sample of (unit, head) pairs -- evenly spaced, plus the first and
last -- over every output and the final state, with the same per-head
tolerance as the scaled tests: max |gpu - ref| <= 2e-4 * max(1, max |ref|).
"""
from __future__ import annotations

import numpy as np
import pytest

from linear_attention_recurrent_gated_amd import workloads as W

from gpu_harness import assert_parity, log, run_case

pytestmark = pytest.mark.gpu


def _sample(wl: W.Workload, n: int = 48) -> np.ndarray:
    P = wl.units_total * wl.heads
    return np.unique(np.concatenate([np.linspace(0, P - 1, n).round().astype(np.int64), [0, P - 1]]))


CASES = [
    # (workload, L, timed steps after any ragged prefix)
    (W.GDN_HYBRID, 16, 2 * 16 + 5),
    (W.KDA_SWEEP, 1, 12),
    (W.KDA_SWEEP, 16, 16 + 7),
    (W.KDA_SWEEP, 64, 64 + 6),
    (W.GDN_LARGE, 32, 32 + 9),
    (W.RWKV6_ADD, 32, 32 + 9),
    (W.GATED, 16, 16 + 7),
]


@pytest.mark.parametrize("wl,L,steps", CASES, ids=[f"{w.name}-L{L}" for w, L, _ in CASES])
def test_full_shape_parity(wl, L, steps):
    T = wl.prefix_steps(L) + steps
    pairs = _sample(wl)
    log(f"case full-shape {wl.name} L={L} T={T} sampled pairs={len(pairs)}")
    paths = ("eager", "af", "af-fused") if wl.variant == W.GDN2 else \
        ("eager", "log", "log-fused", "af", "af-fused")
    case = run_case(wl, L, paths, steps=T, pairs=pairs)
    assert_parity(case, label=f"{wl.name} L={L}")
