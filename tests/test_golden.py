"""The oracle against hand-derived worked examples (tests/golden/hand_worked.json)."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
VARIANTS = {"gdn": oracle.GDN, "kda": oracle.KDA, "rwkv6": oracle.RWKV6}


def test_hand_worked_examples():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        variant = VARIANTS[case["variant"]]
        S0 = np.array(case["S0"], np.float32)
        steps = case["steps"]
        col = lambda key: np.array([s[key] for s in steps], np.float32)[:, None]
        beta = None if variant == oracle.RWKV6 else col("beta")
        o, S = oracle.run(variant, col("q"), col("k"), col("v"), col("g"), beta, S0[None])
        tol = case["tol"]
        for t, s in enumerate(steps):
            ref_o = np.array(s["o"], np.float64)
            assert np.abs(o[t, 0] - ref_o).max() <= tol * max(1, np.abs(ref_o).max()), (case["variant"], t)
        ref_S = np.array(steps[-1]["S"], np.float64)
        assert np.abs(S[0] - ref_S).max() <= tol * max(1, np.abs(ref_S).max()), case["variant"]
