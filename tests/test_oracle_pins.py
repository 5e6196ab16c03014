"""The float64 oracle and the exact models, pinned to facts they do not compute.

See ``oracle_checks.py`` for the checks on the C oracle; the exact-model
tests here pin the deferred (base + log) algebra and the compact WY form.
"""
from __future__ import annotations

import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import exact

from oracle_checks import ALL_CHECKS, GDN, GDN2, KDA, RWKV6, VARIANTS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


def test_threads_do_not_change_results():
    rng = np.random.default_rng(11)
    T, P, d = 20, 13, 16
    q = rng.standard_normal((T, P, d)).astype(np.float32)
    k = rng.standard_normal((T, P, d)).astype(np.float32)
    v = rng.standard_normal((T, P, d)).astype(np.float32)
    g = (-rng.random((T, P, d))).astype(np.float32)
    beta = rng.random((T, P)).astype(np.float32)
    a = oracle.run(KDA, q, k, v, g, beta, threads=1)
    b = oracle.run(KDA, q, k, v, g, beta, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _rand_fr(rng, n, den=8, lo=-8, hi=8):
    return [Fr(int(x), den) for x in rng.integers(lo, hi + 1, size=n)]


def _exact_case(variant, rng, T, d):
    S0 = [_rand_fr(rng, d, 4) for _ in range(d)]
    qs = [_rand_fr(rng, d) for _ in range(T)]
    ks = [_rand_fr(rng, d) for _ in range(T)]
    vs = [_rand_fr(rng, d) for _ in range(T)]
    if variant == GDN:
        alphas = [Fr(int(x), 8) for x in rng.integers(1, 9, size=T)]
    else:
        alphas = [[Fr(int(x), 8) for x in rng.integers(1, 9, size=d)] for _ in range(T)]
    if variant == GDN2:
        betas = [([Fr(int(x), 8) for x in rng.integers(0, 9, size=d)],
                  [Fr(int(x), 8) for x in rng.integers(0, 9, size=d)]) for _ in range(T)]
    else:
        betas = None if variant == RWKV6 else [Fr(int(x), 8) for x in rng.integers(0, 9, size=T)]
    return S0, qs, ks, vs, alphas, betas


WY_VARIANTS = (GDN, KDA, RWKV6)     # the compact-WY log is built for these


@pytest.mark.parametrize("variant", WY_VARIANTS)
@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_deferred_equals_eager_exactly(variant, L):
    """Base + log with q-chain readout and WY merge == the eager recurrence, exactly."""
    rng = np.random.default_rng(100 + 10 * variant + L)
    T, d = 8, 3
    S0, qs, ks, vs, alphas, betas = _exact_case(variant, rng, T, d)
    o_e, S_e = exact.run_stepwise(variant, S0, qs, ks, vs, alphas, betas)
    o_d, S_d, fill = exact.deferred_run(variant, S0, qs, ks, vs, alphas, betas, L)
    assert o_d == o_e
    assert S_d == S_e
    assert fill == T % L


@pytest.mark.parametrize("variant", WY_VARIANTS)
def test_wy_merge_matches_replay(variant):
    """One WY merge of n entries equals n eager steps from the base, exactly."""
    rng = np.random.default_rng(200 + variant)
    n, d = 6, 4
    S0, qs, ks, vs, alphas, betas = _exact_case(variant, rng, n, d)
    log = [(ks[j], vs[j], alphas[j], None if betas is None else betas[j]) for j in range(n)]
    _, S_e = exact.run_stepwise(variant, S0, qs, ks, vs, alphas, betas)
    assert exact.wy_merge(variant, S0, log) == S_e


def test_compact_wy_product():
    """prod_j (I - beta_j k_j k_j^T) = I - K T K^T with T from forward accumulation."""
    rng = np.random.default_rng(12)
    n, d = 5, 4
    ks = [_rand_fr(rng, d) for _ in range(n)]
    betas = [Fr(int(x), 8) for x in rng.integers(0, 17, size=n)]
    P = exact.eye(d)
    for b, k in zip(betas, ks):
        P = exact.matmul(P, exact.madd(exact.eye(d), exact.outer(k, k), -b))
    T = exact.compact_wy_T(betas, ks)
    K = [[ks[j][i] for j in range(n)] for i in range(d)]       # d x n
    KT = [list(k) for k in ks]                                  # n x d
    rhs = exact.madd(exact.eye(d), exact.matmul(exact.matmul(K, T), KT), Fr(-1))
    assert P == rhs
    assert all(T[i][j] == 0 for i in range(n) for j in range(i))


@pytest.mark.parametrize("L", [1, 4, 7, 32])
def test_schedule_closed_form(L):
    for offset in range(L):
        sched = exact.schedule(L, offset, 3 * L + 5)
        for t, (slot, merged, fill) in enumerate(sched):
            assert slot == (offset + t) % L
            assert merged == ((offset + t + 1) % L == 0)
            assert fill == (offset + t + 1) % L


def test_exact_model_matches_oracle_on_floats():
    """The exact stepwise model and the float64 oracle agree on the same float inputs."""
    rng = np.random.default_rng(13)
    T, d = 5, 4
    for variant in VARIANTS:
        S0 = (rng.integers(-4, 5, size=(d, d)) / 4).astype(np.float32)
        q, k, v = ((rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float32) for _ in range(3))
        g = (-rng.integers(0, 5, size=(T,) if variant == GDN else (T, d)) / 8).astype(np.float32)
        if variant == GDN2:
            beta = (rng.integers(0, 9, size=(T, 2 * d)) / 8).astype(np.float32)
            b_exact = [([Fr(float(x)) for x in b[:d]], [Fr(float(x)) for x in b[d:]]) for b in beta]
        else:
            beta = None if variant == RWKV6 else (rng.integers(0, 9, size=T) / 8).astype(np.float32)
            b_exact = None if beta is None else [Fr(float(b)) for b in beta]
        if variant == GDN:
            alphas = [Fr(math.exp(float(x))) for x in g]
        else:
            alphas = [[Fr(math.exp(float(x))) for x in row] for row in g]
        fr = lambda a: [[Fr(float(x)) for x in row] for row in a]
        o_x, S_x = exact.run_stepwise(variant, fr(S0), fr(q), fr(k), fr(v), alphas, b_exact)
        o, S = oracle.run(variant, q[:, None], k[:, None], v[:, None],
                          g[:, None], None if beta is None else beta[:, None], S0[None])
        Sx = np.array([[float(x) for x in r] for r in S_x])
        assert np.abs(S[0] - Sx).max() <= 1e-12 * max(1, np.abs(Sx).max())


@pytest.mark.parametrize("variant", WY_VARIANTS)
@pytest.mark.parametrize("n", [1, 2, 3, 6])
def test_wy_readout_equals_chain_readout(variant, n):
    """The compact-WY readout (R = (I + N)^{-1}, no sequential chain) equals the
    q-chain readout and the eager state's readout, exactly."""
    rng = np.random.default_rng(300 + 10 * variant + n)
    d = 4
    S0, qs, ks, vs, alphas, betas = _exact_case(variant, rng, n, d)
    log = [(ks[j], vs[j], alphas[j], None if betas is None else betas[j]) for j in range(n)]
    q = qs[-1]
    o_wy = exact.wy_readout(variant, S0, log, q)
    assert o_wy == exact.qchain_readout(variant, S0, log, q)
    _, S_e = exact.run_stepwise(variant, S0, qs, ks, vs, alphas, betas)
    assert o_wy == exact.matvec(S_e, q)


@pytest.mark.parametrize("variant", [GDN, KDA])
def test_wy_r_is_inverse_of_unit_triangular(variant):
    """R built one column per appended entry is (I + N)^{-1}."""
    rng = np.random.default_rng(400 + variant)
    n, d = 5, 3
    _, _, ks, vs, alphas, betas = _exact_case(variant, rng, n, d)
    log = [(ks[j], vs[j], alphas[j], betas[j]) for j in range(n)]
    R = exact.wy_build_r(variant, log)
    Nm = [[Fr(0)] * n for _ in range(n)]
    for j in range(1, n):
        u = exact.wy_t_column(variant, log, j)
        for i in range(j):
            Nm[i][j] = u[i]
    I_plus_N = exact.madd(exact.eye(n), Nm)
    assert exact.matmul(I_plus_N, R) == exact.eye(n)


# ----------------------------------------------------------------------------
# additive-factor log
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_af_deferred_equals_eager_exactly(variant, L):
    """Base + additive-factor log (append, readout, merge) == the eager recurrence, exactly."""
    rng = np.random.default_rng(500 + 10 * variant + L)
    T, d = 8, 3
    S0, qs, ks, vs, alphas, betas = _exact_case(variant, rng, T, d)
    o_e, S_e = exact.run_stepwise(variant, S0, qs, ks, vs, alphas, betas)
    o_d, S_d, fill, _ = exact.af_deferred_run(variant, S0, qs, ks, vs, alphas, betas, L)
    assert o_d == o_e
    assert S_d == S_e
    assert fill == T % L


@pytest.mark.parametrize("variant", WY_VARIANTS)
def test_af_factors_are_wy_solve_columns(variant):
    """The factors appended step by step equal the columns of the WY merge's
    triangular solve over the same entries: two derivations, one result."""
    rng = np.random.default_rng(600 + variant)
    n, d = 6, 4
    S0, qs, ks, vs, alphas, betas = _exact_case(variant, rng, n, d)
    _, _, _, factors = exact.af_deferred_run(variant, S0, qs, ks, vs, alphas, betas, n + 1)
    log = [(ks[j], vs[j], alphas[j], None if betas is None else betas[j]) for j in range(n)]
    assert factors == exact.wy_solve_u(variant, S0, log)


def test_additive_factor_against_recurrence_and_exact_model():
    """oracle.additive_factor: S_1 - S_0 diag(alpha) = a k^T for one step of the
    C oracle, and a equals the exact model's factor on float inputs."""
    rng = np.random.default_rng(14)
    P, d = 5, 4
    for variant in VARIANTS:
        S0 = rng.standard_normal((P, d, d)).astype(np.float32)
        q, k, v = (rng.standard_normal((1, P, d)).astype(np.float32) for _ in range(3))
        g = (-rng.random((1, P) if variant == GDN else (1, P, d))).astype(np.float32)
        if variant == GDN2:
            beta = rng.random((1, P, 2 * d)).astype(np.float32)
        else:
            beta = None if variant == RWKV6 else rng.random((1, P)).astype(np.float32)
        _, S1 = oracle.run(variant, q, k, v, g, beta, S0)
        a = oracle.additive_factor(variant, S0, k[0], v[0], g[0], None if beta is None else beta[0])
        alpha = np.exp(g[0].astype(np.float64))
        decayed = S0 * (alpha[:, None, None] if variant == GDN else alpha[:, None, :])
        resid = S1 - decayed - a[:, :, None] * k[0].astype(np.float64)[:, None, :]
        assert np.abs(resid).max() <= 1e-12 * max(1.0, np.abs(S1).max())
        # exact model on exactly representable inputs
        S0x = (rng.integers(-4, 5, size=(d, d)) / 4).astype(np.float32)
        kx, vx = ((rng.integers(-8, 9, size=d) / 8).astype(np.float32) for _ in range(2))
        gx = (-rng.integers(0, 5, size=() if variant == GDN else (d,)) / 8).astype(np.float32)
        if variant == GDN2:
            bx = (rng.integers(0, 9, size=2 * d) / 8).astype(np.float32)
            b_exact = ([Fr(float(x)) for x in bx[:d]], [Fr(float(x)) for x in bx[d:]])
        else:
            bx = np.float32(rng.integers(0, 9) / 8)
            b_exact = Fr(float(bx))
        alpha_x = Fr(math.exp(float(gx))) if variant == GDN else [Fr(math.exp(float(x))) for x in gx]
        ax, _, _ = exact.af_append(variant, [[Fr(float(x)) for x in r] for r in S0x], [],
                                   [Fr(float(x)) for x in kx], [Fr(float(x)) for x in vx],
                                   alpha_x, b_exact)
        af = oracle.additive_factor(variant, S0x[None], kx[None], vx[None],
                                    np.asarray(gx)[None], np.asarray([bx]))
        ref = np.array([float(x) for x in ax])
        assert np.abs(af[0] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_gated_af_equals_kda_when_gates_collapse():
    """Additive-factor deferred run of the gated form with both gates equal to
    KDA's scalar beta reproduces KDA's eager run exactly."""
    rng = np.random.default_rng(700)
    T, d = 7, 3
    S0, qs, ks, vs, alphas, betas = _exact_case(KDA, rng, T, d)
    gates = [([b] * d, [b] * d) for b in betas]
    o_k, S_k = exact.run_stepwise(KDA, S0, qs, ks, vs, alphas, betas)
    o_g, S_g, _, _ = exact.af_deferred_run(GDN2, S0, qs, ks, vs, alphas, gates, 3)
    assert o_g == o_k and S_g == S_k
