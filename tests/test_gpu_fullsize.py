"""GPU parity at the workloads' full shapes and full step counts.

Every call runs on the full state set of the workload (all units and heads,
so the launch configuration is the benchmark's: same grids, same per-call
state size and therefore the same cached / streaming choice for the state
traffic), for every step the workload defines (256 for the tiny GDN case
and the ragged 8-layer set after its 31-step prefix, 512 for the GDN,
per-key-decay and gated sets, 1024 for RWKV6).  The ragged set is driven the
way the benchmark drives it: separate merges name only the units whose logs
are full, and steps that merge in place take their rows in the benchmark's
order.  The float64 oracle then checks a sample of (unit, head) pairs --
evenly spaced, plus the first and last -- over every output and the final
state, with the same per-head tolerance as the scaled tests:
max |gpu - ref| <= 2e-4 * max(1, max |ref|).
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


CASES = [(W.GDN_HYBRID, 16)] + [(W.KDA_SWEEP, L) for L in W.KDA_SWEEP.log_lens] + \
        [(W.GDN_LARGE, 32), (W.RWKV6_ADD, 32), (W.GATED, 16)]


@pytest.mark.parametrize("wl,L", CASES, ids=[f"{w.name}-L{L}-full" for w, L in CASES])
def test_full_shape_full_steps_parity(wl, L):
    T = wl.total_steps(L)
    pairs = _sample(wl)
    log(f"case full-shape {wl.name} L={L} T={T} sampled pairs={len(pairs)}")
    paths = ("eager", "af", "af-fused") if wl.variant == W.GDN2 else \
        ("eager", "log", "log-fused", "af", "af-fused")
    case = run_case(wl, L, paths, steps=T, pairs=pairs, bench_schedule=True)
    assert_parity(case, label=f"{wl.name} L={L} T={T}")
