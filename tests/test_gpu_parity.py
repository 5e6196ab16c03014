"""GPU parity: eager and DeltaLog paths against the float64 oracle.

Tolerance: per (unit, head), over all outputs
and over the final state, max |gpu - ref| <= 2e-4 * max(1, max |ref|).
Sizes here span several workgroups, ragged log tails (steps not a multiple
of L) and ragged per-sequence log offsets; full-size cases are in
test_gpu_fullsize.py.
"""
from __future__ import annotations

import numpy as np
import pytest

from linear_attention_recurrent_gated_amd import workloads as W

from gpu_harness import assert_parity, log, run_case

pytestmark = pytest.mark.gpu

PATHS = ("eager", "log", "log-replay", "log-fused", "af", "af-fused")
GATED_PATHS = ("eager", "af", "af-fused")     # the gated form's log is the factor form


def _paths(wl):
    return GATED_PATHS if wl.variant == W.GDN2 else PATHS


def test_tiny_gdn_full_config():
    """The tiny config exactly: 1 head, d = 64, fp32 inputs, zero state, 256 steps, L = 8."""
    wl = W.TINY_GDN
    log(f"case {wl.name} L=8")
    assert_parity(run_case(wl, 8, PATHS), label=wl.name)


SCALED = [
    # (workload, L)
    (W.GDN_HYBRID.scaled(batch=3, heads=5, steps=70), 16),
    (W.GDN_HYBRID.scaled(batch=2, heads=3, steps=23), 1),
    (W.GDN_HYBRID.scaled(batch=2, heads=3, steps=40), 3),
    (W.GDN_HYBRID.scaled(batch=2, heads=2, steps=130), 64),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=75), 1),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=75), 4),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=75), 8),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=75), 16),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=75), 32),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=140), 64),
    (W.GDN_LARGE.scaled(batch=6, layers=2, heads=3, steps=45), 32),
    (W.RWKV6_ADD.scaled(batch=4, heads=5, steps=100), 32),
    # the other dtype / width combinations the library builds
    (W.KDA_SWEEP.scaled(d_k=64, d_v=64, dtype="f32", batch=2, heads=2, steps=40), 8),
    (W.RWKV6_ADD.scaled(d_k=128, d_v=128, batch=2, heads=2, steps=50), 16),
    (W.GDN_HYBRID.scaled(d_k=64, d_v=64, batch=2, heads=2, steps=50), 16),
    (W.GDN_HYBRID.scaled(dtype="f32", batch=2, heads=2, steps=50), 16),
    (W.RWKV6_ADD.scaled(dtype="f32", batch=2, heads=2, steps=50), 7),
    # fp32 keys with per-channel decay and L = 64 stage 65.5 KiB of LDS (> 64 KiB)
    (W.KDA_SWEEP.scaled(dtype="f32", batch=1, heads=2, steps=70), 64),
    # the gated form (channel-wise erase and write gates)
    (W.GATED.scaled(batch=3, heads=3, steps=70), 16),
    (W.GATED.scaled(batch=2, heads=3, steps=45), 1),
    (W.GATED.scaled(batch=2, heads=2, steps=75), 32),
    (W.GATED.scaled(batch=2, heads=2, steps=140), 64),
    (W.GATED.scaled(d_k=64, d_v=64, dtype="f32", batch=2, heads=2, steps=40), 7),
]


@pytest.mark.parametrize("wl,L", SCALED, ids=[f"{w.name}-{w.variant}-{w.dtype}-d{w.d_k}-L{L}-T{w.steps}"
                                             for w, L in SCALED])
def test_scaled_parity(wl, L):
    log(f"case {wl.name} variant={wl.variant} dtype={wl.dtype} d={wl.d_k} L={L} T={wl.steps}")
    assert_parity(run_case(wl, L, _paths(wl)), label=f"{wl.name} L={L}")


def test_merge_every_step_is_a_no_op_until_full():
    """Calling the full-log merge after every step changes nothing but rounding order."""
    wl = W.GDN_HYBRID.scaled(batch=2, heads=2, steps=37)
    log("case merge-every-step")
    assert_parity(run_case(wl, 8, ("log",), merge_every_step=True), label="merge-every-step")


def test_determinism_bitwise():
    wl = W.KDA_SWEEP.scaled(batch=2, heads=4, steps=41)
    log("case determinism")
    a = run_case(wl, 8, PATHS, run_oracle=False)
    b = run_case(wl, 8, PATHS, run_oracle=False)
    for path in PATHS:
        assert np.array_equal(a.gpu[path][0], b.gpu[path][0]), path
        assert np.array_equal(a.gpu[path][1], b.gpu[path][1]), path


def _random_cases(n=14, seed=2024):
    """Seeded draws over the built shapes: variant, d, dtype, L, batch, heads,
    steps (ragged tails included) and ragged log offsets."""
    rng = np.random.default_rng(seed)
    bases = [W.GDN_HYBRID, W.KDA_SWEEP, W.RWKV6_ADD, W.GATED]
    out = []
    for i in range(n):
        base = bases[i % len(bases)]
        d = int(rng.choice([64, 128]))
        L = int(rng.choice([1, 2, 5, 8, 13, 16, 24, 32, 47, 64]))
        steps = int(rng.integers(L // 2 + 1, 2 * L + 9))
        wl = base.scaled(name=f"{base.name}-rand{i}", d_k=d, d_v=d,
                         dtype=str(rng.choice(["bf16", "f32"])),
                         batch=int(rng.integers(1, 4)), heads=int(rng.integers(1, 4)),
                         steps=steps, ragged=bool(rng.random() < 0.4),
                         state_std=float(rng.choice([0.0, 0.02, 0.5])))
        out.append((wl, L))
    return out


RANDOM = _random_cases()


@pytest.mark.parametrize("wl,L", RANDOM, ids=[f"{w.name}-{w.variant}-{w.dtype}-d{w.d_k}-L{L}-T{w.steps}"
                                             f"{'-ragged' if w.ragged else ''}" for w, L in RANDOM])
def test_random_shapes_parity(wl, L):
    log(f"case {wl.name} variant={wl.variant} dtype={wl.dtype} d={wl.d_k} L={L} T={wl.steps} "
        f"ragged={wl.ragged} std={wl.state_std}")
    assert_parity(run_case(wl, L, _paths(wl)), label=f"{wl.name} L={L}")
