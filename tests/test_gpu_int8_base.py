"""GPU parity of the INT8 base (DL_BASE_I8) against the float64 oracle.

The quantiser is one fp32 decision per entry on both sides, so importing the
same fp32 states must give the same codes, scales and kept values bit for
bit.  A merge quantises the fp32 state the kernel computed, which differs
from the oracle's float64 state in its last bits: codes then agree except
where the oracle's ``S / scale`` lies within 1e-3 of a half-integer (a
rounding boundary), where the neighbouring code is accepted.  To keep every
step's comparison sharp, the run is re-synchronised at each merge: the
oracle's own quantised base is written into the GPU state (oracle values
flow to the GPU, never the reverse) before the unit's next step.  Between
merges the outputs must match the float64 recurrence from the dequantised
base within the path's tolerance, max |gpu - ref| <= 2e-4 * max(1, max |ref|)
per head.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from linear_attention_recurrent_gated_amd import binding as B
from linear_attention_recurrent_gated_amd import workloads as W

from gpu_harness import TOL, log, per_pair_error, to_torch

pytestmark = pytest.mark.gpu


def _state(wl, L, fused, M):
    return B.DecodeState(wl.variant, wl.batch, wl.heads, wl.d_k, L, wl.dtype,
                         merge_on_step=fused, log_form=B.DL_LOG_FACTORS,
                         base_format=B.DL_BASE_I8, kept_channels=M)


def _kept(st, wl, M):
    """Per-pair kept-column lists [P, M] from the state's per-head indices."""
    if M == 0:
        return np.zeros((wl.batch * wl.heads, 0), dtype=np.int64)
    idx = st.kept_idx.cpu().numpy().astype(np.int64)             # [H, M]
    return np.tile(idx, (wl.batch, 1))


def _gpu_base(st):
    c = st.base_codes.cpu().numpy().reshape(-1, st.d, st.d)
    s = st.base_scale.cpu().numpy().reshape(-1, st.d)
    h = (st.base_kept.cpu().numpy().reshape(-1, st.d, st.kept_channels) if st.kept_channels
         else np.zeros((c.shape[0], st.d, 0), np.float32))
    return c, s, h


def _write_base(st, pairs, codes, scale, hp):
    """Put the oracle's quantised base of the flat pairs `pairs` into the state."""
    H = st.heads
    for i, p in enumerate(pairs):
        u, h = divmod(int(p), H)
        st.base_codes[u, h] = torch.from_numpy(codes[i]).cuda()
        st.base_scale[u, h] = torch.from_numpy(scale[i]).cuda()
        if st.kept_channels:
            st.base_kept[u, h] = torch.from_numpy(hp[i]).cuda()


def _compare_codes(gpu, ref, X, label):
    """Codes equal except at rounding boundaries of the oracle's state X."""
    gc, gs, gh = gpu
    rc, rs, rh = ref
    band = quant.boundary_elements(X, rs)
    diff = gc.astype(np.int32) - rc.astype(np.int32)
    bad = (diff != 0) & ~(band & (np.abs(diff) <= 1))
    assert not bad.any(), f"{label}: {int(bad.sum())} codes differ away from a rounding boundary"
    assert np.allclose(gs, rs, rtol=1e-5, atol=0), f"{label}: scales"
    # kept values are fp32 entries of the merged state: the state's bar,
    # per pair relative to max(1, max |S|)
    if gh.size:
        scale = np.maximum(1.0, np.abs(X).reshape(len(X), -1).max(axis=1))[:, None, None]
        kdev = float((np.abs(gh.astype(np.float64) - rh) / scale).max())
        assert kdev <= TOL, f"{label}: kept values off by {kdev:.2e}"
    return int((diff != 0).sum()), int(band.sum())


@pytest.mark.parametrize("wl,M", [
    (W.GDN_HYBRID.scaled(batch=3, heads=4, steps=1), 8),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=1), 16),
    (W.TINY_GDN.scaled(batch=2, heads=2, steps=1), 0),
    (W.GATED.scaled(batch=2, heads=2, steps=1, d_k=64, d_v=64), 4),
])
def test_import_export_bit_exact(wl, M):
    st = _state(wl, 4, False, M)
    rng = np.random.default_rng(11)
    P, d = wl.batch * wl.heads, wl.d_k
    X = (rng.standard_normal((P, d, d)) * rng.choice([1e-3, 0.02, 1.0], size=(P, 1, 1))).astype(np.float32)
    X[0, 3] = 0.0                                                  # a zero row
    kept = _kept(st, wl, M)
    if M:
        X[1, :, kept[1, 0]] = 50.0                                 # an outlier in a kept column
        assert np.all(np.diff(kept[0]) > 0) and kept[0, -1] < d
    st.import_base(torch.from_numpy(X.reshape(wl.batch, wl.heads, d, d)).cuda())
    ref = quant.quantize_base(X, kept)
    got = _gpu_base(st)
    assert np.array_equal(got[0], ref[0]), "codes"
    assert np.array_equal(got[1], ref[1]), "scales"
    assert np.array_equal(got[2], ref[2]), "kept values"
    back = st.export_base().cpu().numpy().reshape(P, d, d)
    expect = ref[0].astype(np.float32) * ref[1][:, :, None]
    for p in range(P):
        expect[p][:, kept[p]] = ref[2][p]
    assert np.array_equal(back, expect)
    assert st.check() == 0
    st.close()


def test_bad_kept_indices_are_flagged():
    wl = W.GDN_HYBRID.scaled(batch=2, heads=2, steps=1)
    st = _state(wl, 4, False, 4)
    st.kept_idx[1] = torch.tensor([3, 3, 9, 20], dtype=torch.int32)   # not increasing
    X = torch.ones((2, 2, 128, 128), device="cuda")
    st.import_base(X)
    assert st.check() == B.DL_FLAG_BAD_KEPT
    s = W.draw_step(wl, 0)
    args = [to_torch(x, wl.dtype) for x in (s.q, s.k, s.v)] + [torch.from_numpy(s.g).cuda(),
                                                                torch.from_numpy(s.beta).cuda()]
    o = st.step_log(*args)
    assert torch.isnan(o[:, 1]).all() and not torch.isnan(o[:, 0]).any()
    assert st.check() == B.DL_FLAG_BAD_KEPT
    st.close()


CASES = [
    (W.GDN_HYBRID.scaled(batch=3, heads=4, steps=27), 8, 8),
    (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=21, state_std=0.02), 4, 16),
    (W.GATED.scaled(batch=2, heads=2, steps=19, state_std=0.02), 8, 4),
    (W.TINY_GDN.scaled(batch=2, heads=2, steps=20, state_std=0.5), 5, 0),
    (W.GDN_LARGE.scaled(batch=5, layers=1, heads=2, steps=14), 4, 8),       # ragged logs
    # logs of 17-32 entries (their own kernel builds)
    (W.GDN_HYBRID.scaled(batch=3, heads=4, steps=56), 24, 8),
    (W.GDN_LARGE.scaled(batch=5, layers=1, heads=2, steps=45), 20, 8),      # ragged logs
]


@pytest.mark.parametrize("fused", [False, True], ids=["merge-launched", "merge-in-step"])
@pytest.mark.parametrize("wl,L,M", CASES, ids=[f"{w.name}-L{L}-M{M}" for w, L, M in CASES])
def test_int8_base_parity_resynced_at_merges(wl, L, M, fused):
    H, d, Bt = wl.heads, wl.d_k, wl.batch
    P = Bt * H
    T = wl.total_steps(L)
    first = W.first_active_step(wl, L)                             # [batch]
    st = _state(wl, L, fused, M)
    kept = _kept(st, wl, M)
    S0 = W.initial_state(wl).reshape(P, d, d)
    st.import_base(torch.from_numpy(S0.reshape(Bt, H, d, d)).cuda())
    base = quant.quantize_base(S0, kept)
    assert np.array_equal(_gpu_base(st)[0], base[0]), "imported codes"
    S = quant.dequantize_base(*base, kept)                         # oracle logical states
    fill = np.zeros(Bt, dtype=np.int64)
    flips = bands = merges = 0
    worst = 0.0
    for tau in range(T):
        s = W.draw_step(wl, tau)
        act = np.nonzero(first <= tau)[0]
        if len(act) == 0:
            continue
        sl = act if len(act) < Bt else slice(None)
        args = [to_torch(x[sl], wl.dtype) for x in (s.q, s.k, s.v)]
        args += [torch.from_numpy(np.ascontiguousarray(s.g[sl])).cuda(),
                 torch.from_numpy(np.ascontiguousarray(s.beta[sl])).cuda()]
        slot = None if len(act) == Bt else torch.from_numpy(act.astype(np.int32)).cuda()
        o = st.step_log(*args, slot_idx=slot).cpu().numpy()        # [rows, H, d]
        fill[act] += 1
        merging = act[fill[act] == L]
        if not fused and len(merging):
            st.merge(B.DL_MERGE_FULL, slot_idx=torch.from_numpy(merging.astype(np.int32)).cuda())
        # the oracle: one float64 step for the active units' pairs
        pairs = (act[:, None] * H + np.arange(H)[None, :]).reshape(-1)
        pick = lambda a: np.asarray(a).reshape(P, *np.asarray(a).shape[2:])[pairs][None]
        o_ref, S_new = oracle.run(wl.variant, pick(s.q_f32), pick(s.k_f32), pick(s.v_f32),
                                  pick(s.g), pick(s.beta), threads=1, S0_f64=S[pairs])
        S[pairs] = S_new
        err = per_pair_error(o.reshape(-1, 1, d), o_ref[0].reshape(-1, 1, d))
        worst = max(worst, float(err.max()))
        assert err.max() <= TOL, f"step {tau}: outputs off by {err.max():.3e}"
        if len(merging):
            mp = (merging[:, None] * H + np.arange(H)[None, :]).reshape(-1)
            ref = quant.quantize_base(S[mp].astype(np.float32), kept[mp])
            got = tuple(x[mp] for x in _gpu_base(st))
            f_, b_ = _compare_codes(got, ref, S[mp], f"step {tau}")
            flips, bands, merges = flips + f_, bands + b_, merges + len(mp)
            _write_base(st, mp, *ref)                              # re-synchronise
            S[mp] = quant.dequantize_base(*ref, kept[mp])
            fill[merging] = 0
    assert st.check() == 0
    assert merges > 0
    log(f"  {wl.name} L={L} M={M} fused={fused}: max rel err o {worst:.2e}, "
        f"{merges} pair merges, {flips} boundary code flips of {bands} boundary entries")
    st.close()


def test_int8_base_readout_and_flush():
    """Readout without an update and the final flush on an INT8 base."""
    wl = W.KDA_SWEEP.scaled(batch=2, heads=2, steps=6, state_std=0.02)
    H, d, Bt, L, M = wl.heads, wl.d_k, wl.batch, 8, 8
    P = Bt * H
    st = _state(wl, L, False, M)
    kept = _kept(st, wl, M)
    S0 = W.initial_state(wl).reshape(P, d, d)
    st.import_base(torch.from_numpy(S0.reshape(Bt, H, d, d)).cuda())
    base = quant.quantize_base(S0, kept)
    S = quant.dequantize_base(*base, kept)
    qs, ks, vs, gs, bs = [], [], [], [], []
    for tau in range(wl.steps):
        s = W.draw_step(wl, tau)
        st.step_log(*[to_torch(x, wl.dtype) for x in (s.q, s.k, s.v)],
                    torch.from_numpy(s.g).cuda(), torch.from_numpy(s.beta).cuda())
        for lst, x in ((qs, s.q_f32), (ks, s.k_f32), (vs, s.v_f32), (gs, s.g), (bs, s.beta)):
            lst.append(x.reshape(P, *x.shape[2:]))
    _, S_ref = oracle.run(wl.variant, np.stack(qs), np.stack(ks), np.stack(vs), np.stack(gs),
                          np.stack(bs), threads=1, S0_f64=S)
    s = W.draw_step(wl, 99)
    o = st.readout(to_torch(s.q, wl.dtype)).cpu().numpy().reshape(P, 1, d)
    o_ref = oracle.readout(S_ref, s.q_f32.reshape(P, d)).reshape(P, 1, d)
    assert per_pair_error(o, o_ref).max() <= TOL
    st.merge(B.DL_MERGE_ALL)
    ref = quant.quantize_base(S_ref.astype(np.float32), kept)
    _compare_codes(_gpu_base(st), ref, S_ref, "flush")
    assert int(st.fill.max()) == 0 and st.check() == 0
    st.close()
