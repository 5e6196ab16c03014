"""Pins of ``oracle.readout`` (o = S q without an update).

The readout is the reference of every GPU readout-only parity check, so it is
pinned here against facts it does not compute itself:

* the step-by-step oracle's own last output, which the recurrence defines as
  the readout of the state after the last step (``o_{T-1} = S_T q_{T-1}``);
  ``oracle.run`` is pinned independently (brute force, invariants, closed
  forms in ``oracle_checks.py``);
* the hand-worked GDN example in ``tests/golden/hand_worked.json``, whose
  state is not symmetric, so a transposed product gives other numbers.

Planted mistakes (a transposed contraction, a readout along the wrong axis
of the query batch) must fail one of these checks.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GDN, KDA, RWKV6, GDN2 = 0, 1, 2, 3


def _case(variant, rng, T=6, P=3, dk=4, dv=4):
    q = rng.standard_normal((T, P, dk)).astype(np.float32)
    k = rng.standard_normal((T, P, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, P, dv)).astype(np.float32)
    g = -np.abs(rng.standard_normal((T, P) if variant == GDN else (T, P, dk))).astype(np.float32)
    if variant == GDN2:
        beta = rng.random((T, P, dk + dv)).astype(np.float32)
    elif variant == RWKV6:
        beta = None
    else:
        beta = rng.random((T, P)).astype(np.float32)
    S0 = rng.standard_normal((P, dv, dk)).astype(np.float32)
    return q, k, v, g, beta, S0


def check_last_output(readout):
    """readout(S_T, q_{T-1}) equals the recurrence's last output, every variant."""
    rng = np.random.default_rng(7)
    for variant in (GDN, KDA, RWKV6, GDN2):
        q, k, v, g, beta, S0 = _case(variant, rng)
        o, S = oracle.run(variant, q, k, v, g, beta, S0, threads=1)
        got = readout(S, q[-1])
        assert got.shape == o[-1].shape
        assert np.allclose(got, o[-1], rtol=1e-13, atol=1e-13), (variant, got, o[-1])


def check_golden(readout):
    """The hand-worked GDN step: S1 = [[1.5, 0], [1.5, 1]], q = (1, 1) -> (1.5, 2.5)."""
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    gdn = next(c for c in cases if c["variant"] == "gdn")
    for step in gdn["steps"]:
        S = np.asarray(step["S"], dtype=np.float64)[None]
        q = np.asarray(step["q"], dtype=np.float64)[None]
        assert np.array_equal(readout(S, q)[0], np.asarray(step["o"], dtype=np.float64)), step


CHECKS = [check_last_output, check_golden]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_readout_pin(check):
    check(oracle.readout)


MUTANTS = {
    "transposed": lambda S, q: np.einsum("pij,pi->pj", np.asarray(S, np.float64), np.asarray(q, np.float64)),
    "query-of-first-state": lambda S, q: np.einsum("pij,j->pi", np.asarray(S, np.float64),
                                                   np.asarray(q, np.float64)[0]),
    "rows-reversed": lambda S, q: np.einsum("pij,pj->pi", np.asarray(S, np.float64)[:, ::-1],
                                            np.asarray(q, np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_readout_mutant_is_caught(name):
    failed = []
    for check in CHECKS:
        try:
            check(MUTANTS[name])
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every readout pin"
