"""Pins of the float64 oracle against facts it does not compute itself.

Each ``check_*`` function raises ``AssertionError`` when the oracle library
(``lib_path``, default: the real one) disagrees with an exact brute force, a
closed form, an invariant or a special case of the recurrence.  They are run
by ``test_oracle_pins.py`` on the real oracle and by
``test_oracle_mutants.py`` on deliberately broken copies of it, each of which
must fail at least one check.

Recurrences (state ``S`` is ``d_v x d_k``, ``alpha = exp(g)``):
GDN ``S' = alpha S (I - beta k k^T) + beta v k^T``; KDA the same with
``S diag(alpha)``; RWKV6-style ``S' = S diag(w) + v k^T``; the gated form
``S' = S diag(alpha) (I - (e * k) k^T) + (w * v) k^T`` (erase gate ``e`` on
the key channels, write gate ``w`` on the value channels, passed as
``beta = [e, w]``); readout ``o = S' q``.
"""
from __future__ import annotations

import math
from fractions import Fraction as Fr

import numpy as np

import oracle
from oracle import exact

GDN, KDA, RWKV6, GDN2 = 0, 1, 2, 3
VARIANTS = (GDN, KDA, RWKV6, GDN2)


def _dyadic(rng, shape, den=8, lo=-8, hi=8):
    """Small dyadic rationals, exact in float32."""
    return (rng.integers(lo, hi + 1, size=shape) / den).astype(np.float32)


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _unit_keys(rng, T, d):
    """Unit vectors with entries +-1/sqrt(d) (d a power of 4): exact in float32."""
    s = 1.0 / math.sqrt(d)
    return (rng.choice([-s, s], size=(T, d))).astype(np.float32)


def _run(variant, lib_path, q, k, v, g, beta=None, S0=None, t_start=None, threads=None):
    """Single-state helper: inputs ``[T, d]`` (or ``[T]`` for scalar g/beta)."""
    T = q.shape[0]
    add = (lambda a: None if a is None else np.asarray(a, np.float32)[:, None])
    o, S = oracle.run(variant, add(q), add(k), add(v), add(g), add(beta),
                      None if S0 is None else np.asarray(S0, np.float32)[None],
                      t_start, threads=threads, lib_path=lib_path)
    return o[:, 0], S[0]


def _alpha_exact(variant, g):
    """The float64 decay the oracle forms, as an exact rational."""
    if variant == GDN:
        return Fr(math.exp(float(g)))
    return [Fr(math.exp(float(x))) for x in g]


def _random_case(variant, rng, T, dk, dv):
    S0 = _dyadic(rng, (dv, dk), den=4)
    q = _dyadic(rng, (T, dk))
    k = _dyadic(rng, (T, dk))
    v = _dyadic(rng, (T, dv))
    g = (-rng.integers(0, 9, size=(T,) if variant == GDN else (T, dk)) / 16).astype(np.float32)
    if variant == GDN2:
        beta = (rng.integers(0, 9, size=(T, dk + dv)) / 8).astype(np.float32)
    else:
        beta = None if variant == RWKV6 else (rng.integers(1, 9, size=T) / 8).astype(np.float32)
    return S0, q, k, v, g, beta


def _betas_exact(variant, beta, dk):
    """Write strengths as exact rationals (the gated form: (erase, write) pairs)."""
    if beta is None:
        return None
    if variant == GDN2:
        return [([Fr(float(x)) for x in b[:dk]], [Fr(float(x)) for x in b[dk:]]) for b in beta]
    return [Fr(float(b)) for b in beta]


def _fr_mat(a):
    return [[Fr(float(x)) for x in row] for row in np.asarray(a)]


def _fr_vecs(a):
    return [[Fr(float(x)) for x in row] for row in np.asarray(a)]


def _to_float(m):
    return np.array([[float(x) for x in row] for row in m])


# ---------------------------------------------------------------------------
def check_bruteforce(lib_path=None):
    """Exact stepwise == explicit product-of-transforms; float64 oracle within 1e-12."""
    rng = np.random.default_rng(1)
    for variant in VARIANTS:
        for (T, dk, dv) in ((6, 4, 3), (5, 3, 4)):
            S0, q, k, v, g, beta = _random_case(variant, rng, T, dk, dv)
            alphas = [_alpha_exact(variant, g[t]) for t in range(T)]
            betas = _betas_exact(variant, beta, dk)
            outs_x, S_x = exact.run_stepwise(variant, _fr_mat(S0), _fr_vecs(q), _fr_vecs(k),
                                             _fr_vecs(v), alphas, betas)
            S_brute = exact.run_product_expansion(variant, _fr_mat(S0), _fr_vecs(k),
                                                  _fr_vecs(v), alphas, betas)
            assert S_x == S_brute, f"stepwise != product expansion (variant {variant})"
            o, S = _run(variant, lib_path, q, k, v, g, beta, S0)
            ref_S = _to_float(S_x)
            ref_o = _to_float(outs_x)
            scale = max(1.0, np.abs(ref_S).max())
            assert np.abs(S - ref_S).max() <= 1e-12 * scale, f"state (variant {variant})"
            scale = max(1.0, np.abs(ref_o).max())
            assert np.abs(o - ref_o).max() <= 1e-12 * scale, f"outputs (variant {variant})"


def check_write_invariant(lib_path=None):
    """beta = 1 and a unit key: the new state maps k_t to v_t exactly (any decay)."""
    rng = np.random.default_rng(2)
    T, d = 24, 64
    for variant in (GDN, KDA):
        k = _unit_keys(rng, T, d)
        v = rng.standard_normal((T, d)).astype(np.float32)
        S0 = rng.standard_normal((d, d)).astype(np.float32)
        g = (-rng.random((T,) if variant == GDN else (T, d))).astype(np.float32)
        beta = np.ones(T, np.float32)
        o, _ = _run(variant, lib_path, k, k, v, g, beta, S0)   # read out with q_t = k_t
        assert np.abs(o - v).max() <= 1e-12, f"S_t k_t != v_t (variant {variant})"


def check_identity(lib_path=None):
    """beta = 0 and alpha = 1 leave S unchanged, bit for bit (RWKV6: v = 0, w = 1)."""
    rng = np.random.default_rng(3)
    T, d = 9, 16
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal((T, d)).astype(np.float32)
    k = rng.standard_normal((T, d)).astype(np.float32)
    for variant in VARIANTS:
        g = np.zeros((T,) if variant == GDN else (T, d), np.float32)
        if variant == RWKV6:
            v, beta = np.zeros((T, d), np.float32), None
        elif variant == GDN2:
            v, beta = rng.standard_normal((T, d)).astype(np.float32), np.zeros((T, 2 * d), np.float32)
        else:
            v, beta = rng.standard_normal((T, d)).astype(np.float32), np.zeros(T, np.float32)
        o, S = _run(variant, lib_path, q, k, v, g, beta, S0)
        assert np.array_equal(S, S0.astype(np.float64)), f"state changed (variant {variant})"
        ref_o = q.astype(np.float64) @ S0.astype(np.float64).T
        assert np.abs(o - ref_o).max() <= 1e-12 * max(1, np.abs(ref_o).max())


def check_additive_closed_form(lib_path=None):
    """RWKV6 with w = 1: S_T = S_0 + V^T K and o_t = (S_0 + sum_{m<=t} v_m k_m^T) q_t."""
    rng = np.random.default_rng(4)
    T, dk, dv = 12, 8, 6
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    q = rng.standard_normal((T, dk)).astype(np.float32)
    k = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    g = np.zeros((T, dk), np.float32)
    o, S = _run(RWKV6, lib_path, q, k, v, g, None, S0)
    K, V = k.astype(np.float64), v.astype(np.float64)
    ref = S0.astype(np.float64) + V.T @ K
    assert np.abs(S - ref).max() <= 1e-12 * np.abs(ref).max()
    for t in range(T):
        St = S0.astype(np.float64) + V[: t + 1].T @ K[: t + 1]
        ref_o = St @ q[t].astype(np.float64)
        assert np.abs(o[t] - ref_o).max() <= 1e-12 * max(1, np.abs(ref_o).max())


def check_pure_decay(lib_path=None):
    """beta = 0: S_T = (prod alpha_t) S_0 for GDN, S_0 diag(prod alpha_t) for KDA."""
    rng = np.random.default_rng(5)
    T, d = 10, 8
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal((T, d)).astype(np.float32)
    k = rng.standard_normal((T, d)).astype(np.float32)
    v = rng.standard_normal((T, d)).astype(np.float32)
    beta = np.zeros(T, np.float32)
    g = (-rng.random(T)).astype(np.float32)
    _, S = _run(GDN, lib_path, q, k, v, g, beta, S0)
    ref = np.prod(np.exp(g.astype(np.float64))) * S0.astype(np.float64)
    assert np.abs(S - ref).max() <= 1e-13 * np.abs(ref).max()
    gc = (-rng.random((T, d))).astype(np.float32)
    _, S = _run(KDA, lib_path, q, k, v, gc, beta, S0)
    ref = S0.astype(np.float64) * np.prod(np.exp(gc.astype(np.float64)), axis=0)[None, :]
    assert np.abs(S - ref).max() <= 1e-13 * np.abs(ref).max()


def check_orthonormal_keys(lib_path=None):
    """alpha = beta = 1 with orthonormal keys: S_T = S_0 (I - K^T K) + V^T K, S_T k_j = v_j."""
    rng = np.random.default_rng(6)
    d, T = 16, 10
    H = _hadamard(d) / 4.0
    K = H[rng.permutation(d)[:T]].astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal((T, d)).astype(np.float32)
    beta = np.ones(T, np.float32)
    for variant in (GDN, KDA):
        g = np.zeros((T,) if variant == GDN else (T, d), np.float32)
        _, S = _run(variant, lib_path, q, K, V, g, beta, S0)
        Kd, Vd = K.astype(np.float64), V.astype(np.float64)
        ref = S0.astype(np.float64) @ (np.eye(d) - Kd.T @ Kd) + Vd.T @ Kd
        assert np.abs(S - ref).max() <= 1e-12 * np.abs(ref).max()
        assert np.abs(S @ Kd.T - Vd.T).max() <= 1e-12 * max(1, np.abs(Vd).max())


def check_channel_decay_collapses(lib_path=None):
    """KDA with a decay that is equal across channels is GDN (bit for bit)."""
    rng = np.random.default_rng(7)
    T, d = 11, 16
    S0, q, k, v, _, beta = _random_case(GDN, rng, T, d, d)
    g = (-rng.random(T)).astype(np.float32)
    gk = np.repeat(g[:, None], d, axis=1)
    o1, S1 = _run(GDN, lib_path, q, k, v, g, beta, S0)
    o2, S2 = _run(KDA, lib_path, q, k, v, gk, beta, S0)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2)


def check_reflection_norm(lib_path=None):
    """beta = 2, v = 0, alpha = 1, unit k: a Householder reflection keeps ||S||_F."""
    rng = np.random.default_rng(8)
    T, d = 16, 64
    k = _unit_keys(rng, T, d)
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    beta = np.full(T, 2.0, np.float32)
    v = np.zeros((T, d), np.float32)
    for variant in (GDN, KDA):
        g = np.zeros((T,) if variant == GDN else (T, d), np.float32)
        _, S = _run(variant, lib_path, k, k, v, g, beta, S0)
        n0 = np.linalg.norm(S0.astype(np.float64))
        assert abs(np.linalg.norm(S) - n0) <= 1e-12 * n0
        assert np.abs(S - S0).max() > 1e-3   # the reflections did act


def check_readout_after_update(lib_path=None):
    """o_t is read from the updated state: o_{T-1} = S_T q_{T-1}."""
    rng = np.random.default_rng(9)
    T, d = 7, 8
    for variant in VARIANTS:
        S0, q, k, v, g, beta = _random_case(variant, rng, T, d, d)
        o, S = _run(variant, lib_path, q, k, v, g, beta, S0)
        ref = S @ q[-1].astype(np.float64)
        assert np.abs(o[-1] - ref).max() <= 1e-13 * max(1, np.abs(ref).max())


def check_late_start(lib_path=None):
    """A state that joins at step t0 equals a run of the remaining steps."""
    rng = np.random.default_rng(10)
    T, d, P = 9, 8, 3
    for variant in VARIANTS:
        cases = [_random_case(variant, rng, T, d, d) for _ in range(P)]
        stack = lambda i: None if cases[0][i] is None else np.stack([c[i] for c in cases], 1)
        S0 = np.stack([c[0] for c in cases])
        t0 = np.array([0, 3, 8], np.int32)
        o, S = oracle.run(variant, stack(1), stack(2), stack(3), stack(4), stack(5), S0, t0,
                          lib_path=lib_path)
        for p in range(P):
            c = cases[p]
            sl = slice(int(t0[p]), T)
            o1, S1 = _run(variant, lib_path, c[1][sl], c[2][sl], c[3][sl], c[4][sl],
                          None if c[5] is None else c[5][sl], c[0])
            assert np.array_equal(S[p], S1)
            assert np.array_equal(o[sl, p], o1) and not o[: int(t0[p]), p].any()


def check_gates_collapse_to_kda(lib_path=None):
    """The gated form with erase and write gates equal to one scalar beta is KDA."""
    rng = np.random.default_rng(11)
    T, d = 10, 16
    S0, q, k, v, g, beta = _random_case(KDA, rng, T, d, d)
    gates = np.repeat(beta[:, None], 2 * d, axis=1)
    o1, S1 = _run(KDA, lib_path, q, k, v, g, beta, S0)
    o2, S2 = _run(GDN2, lib_path, q, k, v, g, gates, S0)
    assert np.abs(S1 - S2).max() <= 1e-13 * max(1, np.abs(S1).max())
    assert np.abs(o1 - o2).max() <= 1e-13 * max(1, np.abs(o1).max())


def check_gated_no_erase(lib_path=None):
    """Erase gate 0: S_T = S_0 diag(P_T) + sum_t (w_t * v_t)(k_t * P_T / P_t)^T, P_t = prod_{m<=t} alpha_m."""
    rng = np.random.default_rng(12)
    T, dk, dv = 9, 8, 6
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    q = rng.standard_normal((T, dk)).astype(np.float32)
    k = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    g = (-rng.random((T, dk))).astype(np.float32)
    w = rng.random((T, dv)).astype(np.float32)
    gates = np.concatenate([np.zeros((T, dk), np.float32), w], axis=1)
    _, S = _run(GDN2, lib_path, q, k, v, g, gates, S0)
    P = np.cumprod(np.exp(g.astype(np.float64)), axis=0)
    ref = S0.astype(np.float64) * P[-1][None, :]
    for t in range(T):
        ref += np.outer(w[t].astype(np.float64) * v[t], k[t].astype(np.float64) * P[-1] / P[t])
    assert np.abs(S - ref).max() <= 1e-12 * np.abs(ref).max()


def check_gated_write_invariant(lib_path=None):
    """Both gates 1, unit key: S_t k_t = v_t for any per-key decay."""
    rng = np.random.default_rng(13)
    T, d = 20, 64
    k = _unit_keys(rng, T, d)
    v = rng.standard_normal((T, d)).astype(np.float32)
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    g = (-rng.random((T, d))).astype(np.float32)
    o, _ = _run(GDN2, lib_path, k, k, v, g, np.ones((T, 2 * d), np.float32), S0)
    assert np.abs(o - v).max() <= 1e-12


ALL_CHECKS = [check_bruteforce, check_write_invariant, check_identity,
              check_additive_closed_form, check_pure_decay, check_orthonormal_keys,
              check_channel_decay_collapses, check_reflection_norm,
              check_readout_after_update, check_late_start, check_gates_collapse_to_kda,
              check_gated_no_erase, check_gated_write_invariant]
