"""The seeded input generator: storage rounding, normalisation, distributions."""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy import integrate, stats

from linear_attention_recurrent_gated_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(10_000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40], np.float32),
        # exact ties between two bf16 values (low 16 bits == 0x8000)
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    ref_back = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref_back)


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 5, 6])
def test_step_shapes_and_norms(cfg_id):
    wl = W.WORKLOADS[cfg_id].scaled(batch=4)
    s = W.draw_step(wl, 3, seed=0)
    U, H = wl.units_total, wl.heads
    assert s.q.shape == (U, H, wl.d_k) and s.v.shape == (U, H, wl.d_v)
    assert s.g.dtype == np.float32
    assert s.g.shape == ((U, H, wl.d_k) if wl.channel_decay else (U, H))
    assert (s.beta is None) == (not wl.has_beta)
    if s.beta is not None:
        assert s.beta.shape == ((U, H) if wl.beta_width == 1 else (U, H, wl.d_k + wl.d_v))
    if wl.dtype == "bf16":
        assert s.q.dtype == np.uint16
        assert np.array_equal(W.bf16_bits_to_f32(s.q), s.q_f32)
    else:
        assert s.q.dtype == np.float32 and np.array_equal(s.q, s.q_f32)
    if wl.qk_l2norm:
        tol = 2.0 ** -7 if wl.dtype == "bf16" else 1e-6
        for a in (s.q_f32, s.k_f32):
            n = np.linalg.norm(a.astype(np.float64), axis=-1)
            assert np.abs(n - 1).max() <= tol
    assert np.all(s.g < 0)
    if s.beta is not None:
        assert np.all((s.beta > 0) & (s.beta < 1))


def test_seeded_and_independent_streams():
    wl = W.GDN_HYBRID.scaled(batch=2)
    a, b = W.draw_step(wl, 5, 0), W.draw_step(wl, 5, 0)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.g, b.g)
    c = W.draw_step(wl, 6, 0)
    assert not np.array_equal(a.q, c.q)
    d = W.draw_step(wl, 5, 1)
    assert not np.array_equal(a.q, d.q)
    par = W.draw_steps(wl, range(8), 0, threads=4)
    seq = W.draw_steps(wl, range(8), 0, threads=1)
    for x, y in zip(par, seq):
        assert np.array_equal(x.k, y.k) and np.array_equal(x.v, y.v)


def _mean_of(f, mu, sd):
    val, _ = integrate.quad(lambda x: f(x) * stats.norm.pdf(x, mu, sd), -12 * sd + mu, 12 * sd + mu)
    return val


@pytest.mark.parametrize("cfg_id", [2, 3, 5, 6])
def test_decay_and_beta_distributions(cfg_id):
    wl = W.WORKLOADS[cfg_id].scaled(batch=16)
    s = W.draw_step(wl, 0, 0)
    alpha = np.exp(s.g.astype(np.float64)).ravel()
    if wl.variant == W.RWKV6:
        f = lambda x: np.exp(-np.exp(x))
    else:
        f = lambda x: np.exp(-np.logaddexp(0.0, x))
    mean = _mean_of(f, wl.decay_mean, wl.decay_std)
    se = alpha.std() / np.sqrt(alpha.size)
    assert abs(alpha.mean() - mean) < 5 * se
    if s.beta is not None:
        b = s.beta.astype(np.float64).ravel()
        assert abs(b.mean() - 0.5) < 5 * b.std() / np.sqrt(b.size)
    v = s.v_f32.astype(np.float64).ravel()
    assert abs(v.mean()) < 5 / np.sqrt(v.size) and abs(v.std() - 1) < 0.01


def test_initial_state_and_offsets():
    wl = W.GDN_LARGE.scaled(batch=64, layers=2, heads=2)
    S0 = W.initial_state(wl, 0)
    assert S0.shape == (128, 2, 128, 128) and S0.dtype == np.float32
    assert abs(S0.std() - 0.02) < 0.001
    assert not W.initial_state(W.KDA_SWEEP.scaled(batch=1, heads=1), 0).any()
    L = 32
    f = W.ragged_offsets(wl, L, 0)
    assert f.shape == (64,) and f.min() >= 0 and f.max() < L and len(set(f.tolist())) > 8
    first = W.first_active_step(wl, L, 0)
    assert np.array_equal(first, L - 1 - f)
    for tau in range(wl.prefix_steps(L) + 2):
        rows = W.active_rows(wl, L, tau, 0)
        assert np.array_equal(rows, np.nonzero(first <= tau)[0])
    assert len(W.active_rows(wl, L, L - 1, 0)) == 64
    flat = W.TINY_GDN
    assert flat.prefix_steps(8) == 0 and not W.first_active_step(flat, 8).any()
