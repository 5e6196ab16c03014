"""Pins of the mixed-precision base oracle (``oracle/quant.py``): INT8 codes
with one fp32 scale per value row and fp32 kept key channels.

The quantiser is pinned against values whose codes are known without it:
states on the INT8 grid of a power-of-two scale (every division exact),
ties that must go to the even code, the error bound of round-to-nearest,
all-zero rows, and kept columns that must neither enter the scale nor lose
a bit.  Planted mistakes (a per-column scale, ties away from zero, kept
columns inside the scale, a 128-step grid, no clip) must each fail a pin.
The mixed recurrence is pinned to the plain float64 oracle (no merge inside
the run, a base already on the grid) and to the schedule model of the
deferred log (a merge after every L-th step of a state, counted from its
first).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import exact, quant

GDN, KDA = 0, 1
S7 = np.float32(2.0 ** -7)


def _grid_state(rng, P, dv, dk, kept):
    """States on the INT8 grid of scale 2^-7 with a full-scale entry in every
    row (outside the kept columns), kept columns holding arbitrary fp32."""
    codes = rng.integers(-127, 128, size=(P, dv, dk))
    free = [j for j in range(dk) if j not in kept]
    codes[:, np.arange(dv), rng.choice(free, size=dv)] = rng.choice([-127, 127], size=(P, dv))
    X = (codes * S7).astype(np.float32)
    X[:, :, kept] = rng.standard_normal((P, dv, len(kept))).astype(np.float32)
    codes[:, :, kept] = 0
    return X, codes.astype(np.int8)


def check_grid_round_trip(qz):
    rng = np.random.default_rng(1)
    kept = [2, 9]
    X, codes = _grid_state(rng, 3, 6, 12, kept)
    c, s, h = qz(X, np.array([kept] * 3))
    assert np.array_equal(c, codes)
    assert np.all(s == S7)
    assert np.array_equal(h, X[:, :, kept])


def check_ties_to_even(qz):
    row = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], dtype=np.float64)
    X = (row * float(S7)).astype(np.float32)[None, None, :]
    c, s, _ = qz(X, np.array([[7]]))            # the 126.5 entry is kept, not coded
    assert s[0, 0] == S7
    assert c[0, 0].tolist() == [127, 0, 2, 2, 0, -2, -2, 0]


def check_error_bound(qz):
    rng = np.random.default_rng(2)
    X = rng.standard_normal((4, 16, 16)).astype(np.float32) * np.float32(0.05)
    kept = np.array([[0, 5, 11]] * 4)
    c, s, h = qz(X, kept)
    D = quant.dequantize_base(c, s, h, kept)
    mask = np.ones(16, bool)
    mask[kept[0]] = False
    err = np.abs(D - X)[:, :, mask]
    assert np.all(err <= s[:, :, None].astype(np.float64) * (0.5 + 1e-6))
    assert np.array_equal(D[:, :, kept[0]], X[:, :, kept[0]].astype(np.float64))
    amax = np.abs(X[:, :, mask]).max(axis=2)
    assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32))
    assert np.abs(c).max() == 127


def check_zero_rows_and_kept_outliers(qz):
    X = np.zeros((1, 3, 8), dtype=np.float32)
    X[0, 1, :] = np.float32(0.25)
    X[0, :, 3] = np.float32(1e6)                 # an outlier in a kept column
    c, s, h = qz(X, np.array([[3]]))
    assert s[0, 0] == 0 and s[0, 2] == 0 and not c[0, 0].any() and not c[0, 2].any()
    assert s[0, 1] == np.float32(np.float32(0.25) / np.float32(127))
    assert np.all(c[0, 1, [0, 1, 2, 4, 5, 6, 7]] == 127) and c[0, 1, 3] == 0
    assert np.all(h[0, :, 0] == np.float32(1e6))


CHECKS = [check_grid_round_trip, check_ties_to_even, check_error_bound,
          check_zero_rows_and_kept_outliers]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_quantizer_pin(check):
    check(quant.quantize_base)


def _mutant(kind):
    def qz(X, hp_idx):
        X = np.asarray(X, dtype=np.float32)
        P, dv, dk = X.shape
        keep = quant._mask(dk, hp_idx)[:, None, :]
        mag = np.abs(X) if kind == "kept-in-scale" else np.where(keep, 0, np.abs(X))
        if kind == "per-column":
            amax = np.broadcast_to(mag.max(axis=1, keepdims=True), X.shape)
        else:
            amax = np.broadcast_to(mag.max(axis=2, keepdims=True), X.shape)
        qmax = 128 if kind == "grid-128" else 127
        scale = (amax / np.float32(qmax)).astype(np.float32)
        r = X / np.where(scale > 0, scale, 1)
        if kind == "ties-away":
            r = np.sign(r) * np.floor(np.abs(r) + 0.5)
        else:
            r = np.rint(r)
        if kind != "no-clip":
            r = np.clip(r, -127, 127)
        codes = np.where((scale > 0) & ~keep, r, 0).astype(np.int8 if kind != "no-clip" else np.int16)
        hp = np.take_along_axis(X, np.broadcast_to(np.asarray(hp_idx)[:, None, :],
                                                   (P, dv, np.asarray(hp_idx).shape[1])), axis=2)
        return codes, scale[:, :, 0].astype(np.float32), hp
    return qz


@pytest.mark.parametrize("kind", ["per-column", "kept-in-scale", "grid-128", "ties-away"])
def test_quantizer_mutant_is_caught(kind):
    failed = []
    for check in CHECKS:
        try:
            check(_mutant(kind))
        except (AssertionError, IndexError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {kind} passed every quantiser pin"


def _inputs(rng, T, P, d, variant):
    q = rng.standard_normal((T, P, d)).astype(np.float32)
    k = rng.standard_normal((T, P, d))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((T, P, d)).astype(np.float32)
    g = -np.abs(rng.standard_normal((T, P) if variant == GDN else (T, P, d))).astype(np.float32)
    b = rng.random((T, P)).astype(np.float32)
    return q, k, v, g, b


@pytest.mark.parametrize("variant", [GDN, KDA])
def test_no_merge_on_grid_is_the_plain_recurrence(variant):
    """A base already on the grid and no merge inside the run: exactly the
    float64 recurrence from that base."""
    rng = np.random.default_rng(3)
    T, P, d = 7, 3, 8
    q, k, v, g, b = _inputs(rng, T, P, d, variant)
    kept = np.array([[1, 6]] * P)
    S0, _ = _grid_state(rng, P, d, d, [1, 6])
    o, S, _ = quant.run_quantized_base(variant, q, k, v, g, b, S0, None, T + 1, kept)
    o2, S2 = oracle.run(variant, q, k, v, g, b, S0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


@pytest.mark.parametrize("L,offset", [(1, 0), (3, 0), (4, 2), (5, 4)])
def test_merges_follow_the_log_schedule(L, offset):
    """The base is re-quantised exactly where the deferred log merges: a step
    whose output is unchanged by quantising the state before it follows a
    merge iff the schedule model says one happened; checked through the
    outputs of a run that is split and resumed at those points."""
    rng = np.random.default_rng(4 + L)
    T, P, d = 3 * L + 2, 2, 8
    q, k, v, g, b = _inputs(rng, T, P, d, GDN)
    kept = np.array([[0, 3]] * P)
    S0 = (rng.standard_normal((P, d, d)) * 0.3).astype(np.float32)
    t_start = np.array([offset, 0])
    o, _, _ = quant.run_quantized_base(GDN, q, k, v, g, b, S0, t_start, L, kept)
    # rebuild pair 0 from the schedule model: plain float64 segments between
    # the merges the model lists, quantising at each
    sched = exact.schedule(L, 0, T - offset)
    S = quant.dequantize_base(*quant.quantize_base(S0[:1], kept[:1]), kept[:1])
    t = offset
    ref = np.zeros((T, d))
    start = t
    for i, (_, merged, _) in enumerate(sched):
        if merged or i == len(sched) - 1:
            seg = slice(start, offset + i + 1)
            os_, S = oracle.run(GDN, q[seg][:, :1], k[seg][:, :1], v[seg][:, :1], g[seg][:, :1],
                                b[seg][:, :1], threads=1, S0_f64=S)
            ref[seg] = os_[:, 0]
            if merged:
                S = quant.dequantize_base(*quant.quantize_base(S.astype(np.float32), kept[:1]), kept[:1])
            start = offset + i + 1
    assert np.array_equal(o[:, 0], ref)
    assert not o[:offset, 0].any()
    # and the merges do change the run: without them it differs
    o_plain, _ = oracle.run(GDN, q[:, :1], k[:, :1], v[:, :1], g[:, :1], b[:, :1],
                            S0_f64=quant.dequantize_base(*quant.quantize_base(S0[:1], kept[:1]), kept[:1]),
                            t_start=t_start[:1])
    if T - offset > L:
        assert not np.array_equal(o[:, 0], o_plain[:, 0])


def test_float64_initial_state_entry():
    """oracle.run with a float64 initial state equals the fp32 entry when the
    state is an fp32 value, and keeps the bits of one that is not."""
    rng = np.random.default_rng(5)
    q, k, v, g, b = _inputs(rng, 5, 2, 8, KDA)
    S0 = rng.standard_normal((2, 8, 8)).astype(np.float32)
    o1, S1 = oracle.run(KDA, q, k, v, g, b, S0)
    o2, S2 = oracle.run(KDA, q, k, v, g, b, S0_f64=S0.astype(np.float64))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    # a state between fp32 values: g = 0, beta = 0 leaves it untouched
    Sx = S0.astype(np.float64) * (1 + 2.0 ** -40)
    _, S3 = oracle.run(KDA, q, k, v, np.zeros_like(g), np.zeros_like(b), S0_f64=Sx)
    assert np.array_equal(S3, Sx)


def test_boundary_elements():
    s = np.array([[0.5]])
    X = np.array([[[0.25, 0.2501, 0.3, -0.7499, 0.0]]])   # x/s = 0.5, 0.5002, 0.6, -1.4998, 0
    assert quant.boundary_elements(X, s, band=1e-3).tolist() == [[[True, True, False, True, False]]]
