"""GPU edge cases: the log schedule bit for bit, readout, device flags,
slot mapping, argument checks that need a live state."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_gated_amd import binding as B
from linear_attention_recurrent_gated_amd import workloads as W

from gpu_harness import TOL, log, per_pair_error, run_case, to_torch

pytestmark = pytest.mark.gpu


def _inputs(wl, tau, rows=None):
    s = W.draw_step(wl, tau)
    sl = slice(None) if rows is None else rows
    q, k, v = (to_torch(x[sl], wl.dtype) for x in (s.q, s.k, s.v))
    g = torch.from_numpy(np.ascontiguousarray(s.g[sl])).cuda()
    beta = None if s.beta is None else torch.from_numpy(np.ascontiguousarray(s.beta[sl])).cuda()
    return s, (q, k, v, g, beta)


def _beta_rows(wl, s, P):
    """Write strengths of one step per (unit, head): [P] or, gated, [P, d_k + d_v]."""
    return s.beta.reshape((P,) if wl.beta_width == 1 else (P, -1))


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("wl,L", [
    (W.GDN_LARGE.scaled(batch=5, layers=1, heads=2, steps=14), 4),
    (W.KDA_SWEEP.scaled(batch=3, heads=2, steps=11, ragged=True), 3),
    (W.RWKV6_ADD.scaled(batch=3, heads=2, steps=9, ragged=True), 5),
])
@pytest.mark.parametrize("path", ["log", "log-fused"])
def test_schedule_and_payload_bit_exact(wl, L, path):
    """After every step: fill == (tokens so far) mod L for every head, and the
    slot written holds bit copies of that step's k, v and beta, and the decay
    accumulated through it."""
    first = W.first_active_step(wl, L)
    log(f"case schedule {wl.name} L={L} offsets={L - 1 - first}")

    def on_step(tau, states):
        st = states[path][0]
        s = W.draw_step(wl, tau)
        fill = st.fill.cpu().numpy()
        for b in range(wl.batch):
            m = tau - first[b] + 1                      # tokens this sequence has taken
            expect = max(m, 0) % L
            assert np.all(fill[b] == expect), (tau, b, fill[b], expect)
            if m <= 0 or (path.endswith("-fused") and m % L == 0):
                continue                                # merged in place: no entry kept
            slot = (m - 1) % L
            assert np.array_equal(_bits(st.log_k[b, :, slot]), _bits(to_torch(s.k[b], wl.dtype)))
            assert np.array_equal(_bits(st.log_v[b, :, slot]), _bits(to_torch(s.v[b], wl.dtype)))
            # the log keeps the decay accumulated since its first entry, summed in
            # fp32 in entry order
            lam = np.zeros_like(s.g[b])
            for tp in range(tau - slot, tau + 1):
                lam = (lam + W.draw_step(wl, tp).g[b]).astype(np.float32)
            assert np.array_equal(st.log_g[b, :, slot].cpu().numpy(), lam)
            if s.beta is not None:
                assert np.array_equal(st.log_beta[b, :, slot].cpu().numpy(), s.beta[b])

    run_case(wl, L, (path,), merge_every_step=True, run_oracle=False, on_step=on_step)


@pytest.mark.parametrize("wl,L", [
    (W.GDN_LARGE.scaled(batch=5, layers=1, heads=2, steps=14), 4),
    (W.KDA_SWEEP.scaled(batch=3, heads=2, steps=11, ragged=True), 3),
    (W.GDN_HYBRID.scaled(d_k=64, d_v=64, dtype="f32", batch=2, heads=3, steps=10), 4),
    (W.GATED.scaled(batch=3, heads=2, steps=9), 4),
])
@pytest.mark.parametrize("path", ["af", "af-fused"])
def test_factor_log_payload(wl, L, path):
    """Additive-factor log after every step: fill == (tokens so far) mod L,
    the slot written holds a bit copy of k, the decay accumulated through it
    (fp32, entry order), and the factor a_t = beta (v - S_{t-1}(alpha k))
    within the parity tolerance of the oracle's factor."""
    first = W.first_active_step(wl, L)
    H, d = wl.heads, wl.d_k
    P = wl.batch * H
    S0 = W.initial_state(wl).reshape(P, d, d)
    t_start = np.repeat(first, H)
    hist = []
    log(f"case factor payload {wl.name} L={L} {path}")

    def on_step(tau, states):
        st = states[path][0]
        s = W.draw_step(wl, tau)
        hist.append(s)
        if tau > 0:
            stack = lambda f: np.stack([f(x) for x in hist[:-1]])
            _, S_prev = oracle.run(wl.variant, stack(lambda x: x.q_f32.reshape(P, d)),
                                   stack(lambda x: x.k_f32.reshape(P, d)),
                                   stack(lambda x: x.v_f32.reshape(P, d)),
                                   stack(lambda x: x.g.reshape(P, -1) if wl.channel_decay else x.g.reshape(P)),
                                   stack(lambda x: _beta_rows(wl, x, P)), S0, t_start)
        else:
            S_prev = S0.astype(np.float64)
        a_ref = oracle.additive_factor(wl.variant, S_prev, s.k_f32.reshape(P, d), s.v_f32.reshape(P, d),
                                       s.g.reshape(P, -1) if wl.channel_decay else s.g.reshape(P),
                                       _beta_rows(wl, s, P)).reshape(wl.batch, H, d)
        fill = st.fill.cpu().numpy()
        for b in range(wl.batch):
            m = tau - first[b] + 1
            assert np.all(fill[b] == max(m, 0) % L), (tau, b, fill[b])
            if m <= 0 or (path.endswith("-fused") and m % L == 0):
                continue                                # merged in place: no entry kept
            slot = (m - 1) % L
            assert np.array_equal(_bits(st.log_k[b, :, slot]), _bits(to_torch(s.k[b], wl.dtype)))
            lam = np.zeros_like(s.g[b])
            for tp in range(tau - slot, tau + 1):
                lam = (lam + W.draw_step(wl, tp).g[b]).astype(np.float32)
            assert np.array_equal(st.log_g[b, :, slot].cpu().numpy(), lam)
            a = st.log_v[b, :, slot].double().cpu().numpy()
            e = per_pair_error(a, a_ref[b])
            assert e.max() <= TOL, (tau, b, e.max())

    run_case(wl, L, (path,), merge_every_step=True, run_oracle=False, on_step=on_step)


_READOUT_CASES = [(w, f, 6, (0, 3, 5, 8, 13, 19))
                  for w in (W.GDN_HYBRID.scaled(batch=2, heads=3, steps=20),
                            W.KDA_SWEEP.scaled(batch=2, heads=3, steps=20),
                            W.RWKV6_ADD.scaled(batch=2, heads=3, steps=20),
                            W.GATED.scaled(batch=2, heads=3, steps=20))
                  for f in (B.DL_LOG_WY, B.DL_LOG_FACTORS)
                  if not (w.variant == W.GDN2 and f == B.DL_LOG_WY)]   # gated: factor log only
# per-key decays with a log longer than 32 entries (the WY readout stages its
# entries 32 at a time): readouts with 21, 35 and 39 entries, and after a merge
_READOUT_CASES += [(W.KDA_SWEEP.scaled(batch=2, heads=3, steps=46), f, 40, (20, 34, 38, 45))
                   for f in (B.DL_LOG_WY, B.DL_LOG_FACTORS)]


@pytest.mark.parametrize("wl,form,L,taus", _READOUT_CASES,
                         ids=[f"{('gdn', 'kda', 'rwkv6', 'gated')[w.variant]}-{'factors' if f else 'wy'}-L{L}"
                              for w, f, L, _ in _READOUT_CASES])
def test_readout_matches_oracle(wl, form, L, taus):
    """dl_readout returns S_t q for a fresh q, mid-log and after merges, and changes nothing."""
    H, d = wl.heads, wl.d_k
    P = wl.batch * H
    log(f"case readout {wl.name} form={form}")
    st = B.DecodeState(wl.variant, wl.batch, H, d, L, wl.dtype, log_form=form)
    eg = B.DecodeState(wl.variant, wl.batch, H, d, 0, wl.dtype)
    S0 = W.initial_state(wl)
    st.base.copy_(torch.from_numpy(S0))
    eg.base.copy_(torch.from_numpy(S0))
    rng = np.random.default_rng(5)
    hist = []
    for tau in range(wl.steps):
        s, args = _inputs(wl, tau)
        hist.append(s)
        st.step_log(*args)
        eg.step_eager(*args)
        if (tau + 1) % L == 0:
            st.merge(B.DL_MERGE_FULL)
        if tau in taus:
            qn = rng.standard_normal((wl.batch, H, d))
            qs, qf = W.store(qn, wl.dtype)
            qt = to_torch(qs, wl.dtype)
            before = (st.base.clone(), st.fill.clone())
            o_log = st.readout(qt).double().cpu().numpy().reshape(P, d)
            o_eag = eg.readout(qt).double().cpu().numpy().reshape(P, d)
            assert torch.equal(before[0], st.base) and torch.equal(before[1], st.fill)
            T = tau + 1
            stack = lambda f: np.stack([f(x) for x in hist])
            _, S_ref = oracle.run(wl.variant, stack(lambda x: x.q_f32.reshape(P, d)),
                                  stack(lambda x: x.k_f32.reshape(P, d)),
                                  stack(lambda x: x.v_f32.reshape(P, d)),
                                  stack(lambda x: x.g.reshape(P, -1) if wl.channel_decay else x.g.reshape(P)),
                                  None if hist[0].beta is None else stack(lambda x: _beta_rows(wl, x, P)),
                                  S0.reshape(P, d, d))
            ref = oracle.readout(S_ref, qf.reshape(P, d))
            for name, o in (("log", o_log), ("eager", o_eag)):
                e = per_pair_error(o, ref)
                assert e.max() <= TOL, (name, tau, e.max())
    assert st.check() == 0 and eg.check() == 0


@pytest.mark.parametrize("form", [B.DL_LOG_WY, B.DL_LOG_FACTORS], ids=["wy", "factors"])
def test_device_flags(form):
    wl = W.GDN_HYBRID.scaled(batch=2, heads=2, steps=4)
    H, d = wl.heads, wl.d_k
    st = B.DecodeState(wl.variant, 2, H, d, 2, wl.dtype, log_form=form)
    _, args = _inputs(wl, 0)
    st.step_log(*args)
    st.step_log(*args)
    assert st.check() == 0 and int(st.fill.max()) == 2
    base = st.base.clone()
    o = st.step_log(*args)                       # log is full: rejected
    assert torch.isnan(o).all()
    assert st.check() == B.DL_FLAG_LOG_FULL
    assert st.check() == 0                       # check clears the flags
    assert torch.equal(base, st.base) and int(st.fill.max()) == 2
    o = st.step_eager(*args)                     # eager on a non-empty log: rejected
    assert torch.isnan(o).all() and st.check() == B.DL_FLAG_LOG_NONEMPTY
    st.merge(B.DL_MERGE_FULL)
    assert int(st.fill.max()) == 0 and st.check() == 0
    bad = torch.tensor([0, 7], dtype=torch.int32, device="cuda")
    o = st.step_log(*args, slot_idx=bad)
    assert torch.isnan(o[1]).all() and not torch.isnan(o[0]).any()
    assert st.check() == B.DL_FLAG_BAD_SLOT
    st.close()


@pytest.mark.parametrize("form", [B.DL_LOG_WY, B.DL_LOG_FACTORS], ids=["wy", "factors"])
def test_permuted_slots_match_identity(form):
    """Rows map to units through slot_idx in any order."""
    wl = W.KDA_SWEEP.scaled(batch=4, heads=2, steps=9)
    H, d, L = wl.heads, wl.d_k, 4
    a = B.DecodeState(wl.variant, 4, H, d, L, wl.dtype, log_form=form)
    b = B.DecodeState(wl.variant, 4, H, d, L, wl.dtype, log_form=form)
    perm = np.array([2, 0, 3, 1])
    slot = torch.from_numpy(perm.astype(np.int32)).cuda()
    for tau in range(wl.steps):
        _, args = _inputs(wl, tau)
        oa = a.step_log(*args)
        pargs = tuple(None if x is None else x[torch.from_numpy(perm).cuda()].contiguous() for x in args)
        ob = b.step_log(*pargs, slot_idx=slot)
        assert torch.equal(oa[torch.from_numpy(perm).cuda()], ob)
        if (tau + 1) % L == 0:
            a.merge()
            b.merge(rows=4, slot_idx=slot)
    assert torch.equal(a.base, b.base) and torch.equal(a.fill, b.fill)


@pytest.mark.parametrize("path", ["eager", "wy", "wy-fused", "factors", "factors-fused",
                                  "factors-i8", "factors-fused-i8"])
def test_row_order_changes_nothing(path):
    """Workgroups taken in a caller-given row order produce bit-identical
    outputs, states and logs (over an fp32 or an INT8 base); an order entry
    out of range is flagged."""
    wl = W.GDN_LARGE.scaled(batch=7, layers=1, heads=3, steps=11)
    H, d, L, Bt = wl.heads, wl.d_k, 4, wl.batch
    form = B.DL_LOG_FACTORS if path.startswith("factors") else B.DL_LOG_WY
    Lp = 0 if path == "eager" else L
    i8 = path.endswith("-i8")
    fused = "-fused" in path
    kw = dict(base_format=B.DL_BASE_I8, kept_channels=8) if i8 else {}
    a = B.DecodeState(wl.variant, Bt, H, d, Lp, wl.dtype, log_form=form, merge_on_step=fused, **kw)
    b = B.DecodeState(wl.variant, Bt, H, d, Lp, wl.dtype, log_form=form, merge_on_step=fused, **kw)
    S0 = torch.from_numpy(W.initial_state(wl)).cuda()
    if i8:
        a.import_base(S0)
        b.import_base(S0)
    else:
        a.base.copy_(S0)
        b.base.copy_(S0)
    rng = np.random.default_rng(3)
    for tau in range(wl.steps):
        _, args = _inputs(wl, tau)
        order = torch.from_numpy(rng.permutation(Bt).astype(np.int32)).cuda()
        if path == "eager":
            oa = a.step_eager(*args)
            ob = b.step_eager(*args, row_order=order)
        else:
            oa = a.step_log(*args)
            ob = b.step_log(*args, row_order=order)
            if not fused and (tau + 1) % L == 0:
                a.merge()
                b.merge()
        assert torch.equal(oa, ob), f"outputs differ at step {tau}"
    assert torch.equal(a.buf, b.buf)
    assert a.check() == 0 and b.check() == 0
    bad = torch.tensor([0, 1, 2, 3, 4, 5, 9], dtype=torch.int32, device="cuda")
    _, args = _inputs(wl, wl.steps)
    fill = b.fill.clone()
    if path == "eager":
        o = b.step_eager(*args, row_order=bad)
    else:
        o = b.step_log(*args, row_order=bad)
    assert b.check() == B.DL_FLAG_BAD_SLOT
    assert not torch.isnan(o[:6]).any()
    assert path == "eager" or torch.equal(b.fill[6], fill[6])   # row 6 was never served
    a.close()
    b.close()


def test_zero_rows_and_argument_errors():
    wl = W.GDN_HYBRID.scaled(batch=2, heads=2, steps=1)
    H, d = wl.heads, wl.d_k
    st = B.DecodeState(wl.variant, 2, H, d, 4, wl.dtype)
    _, (q, k, v, g, beta) = _inputs(wl, 0)
    o = torch.empty((2, H, d), device="cuda")
    lib = B.load()
    h = st.handle
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.dl_decode_step_log(h, 0, None, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(o), None) == 0
    assert lib.dl_decode_step_log(h, 2, None, ptr(q), ptr(k), ptr(v), ptr(g), None, ptr(o), None) == B.DL_ERR_INVALID
    assert lib.dl_decode_step_log(h, 3, None, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(o), None) == B.DL_ERR_INVALID
    mis = ctypes.c_void_p(q.data_ptr() + 2)
    assert lib.dl_decode_step_eager(h, 2, None, mis, ptr(k), ptr(v), ptr(g), ptr(beta), ptr(o), None) == B.DL_ERR_INVALID
    assert lib.dl_merge(h, 2, None, 5, None) == B.DL_ERR_INVALID
    assert lib.dl_decode_step_log_ordered(h, 2, None, mis, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                                          ptr(o), None) == B.DL_ERR_INVALID   # misaligned order
    e = B.DecodeState(wl.variant, 2, H, d, 0, wl.dtype)
    assert lib.dl_decode_step_log(e.handle, 2, None, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(o), None) == B.DL_ERR_INVALID
    assert st.check() == 0 and int(st.fill.max()) == 0
    st.close()
    e.close()


@pytest.mark.parametrize("wl,L", [(W.GDN_HYBRID.scaled(batch=3, heads=4, steps=16), 16),
                                  (W.KDA_SWEEP.scaled(batch=3, heads=4, steps=64), 64),
                                  (W.RWKV6_ADD.scaled(batch=3, heads=4, steps=32), 32),
                                  (W.KDA_SWEEP.scaled(batch=2, heads=2, steps=13), 13),
                                  (W.GDN_HYBRID.scaled(batch=3, heads=4, steps=37), 48),
                                  (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=41), 64),
                                  (W.KDA_SWEEP.scaled(batch=2, heads=3, steps=16), 64)],
                         ids=["gdn16", "kda64", "rwkv32", "kda13-partial", "gdn48-partial",
                              "kda64-partial", "kda64-one-chunk"])
def test_wy_merge_equals_replay_merge(wl, L):
    """The MFMA WY merge and the step-by-step replay merge agree closely."""
    H, d = wl.heads, wl.d_k
    a = B.DecodeState(wl.variant, wl.batch, H, d, L, wl.dtype)
    b = B.DecodeState(wl.variant, wl.batch, H, d, L, wl.dtype)
    S0 = torch.from_numpy(W.initial_state(wl.scaled(state_std=0.5)))
    a.base.copy_(S0)
    b.base.copy_(S0)
    for tau in range(wl.steps):
        _, args = _inputs(wl, tau)
        a.step_log(*args)
        b.step_log(*args)
    a.merge(B.DL_MERGE_ALL)
    b.merge(B.DL_MERGE_ALL, replay=True)
    x, y = a.base.double().cpu().numpy(), b.base.double().cpu().numpy()
    err = per_pair_error(x.reshape(-1, d, d), y.reshape(-1, d, d)).max()
    log(f"  WY vs replay {wl.name} L={L}: {err:.2e}")
    assert err <= 1e-5
    assert int(a.fill.max()) == 0 and int(b.fill.max()) == 0


def _degenerate_inputs(variant, U, H, d, T, seed=11):
    """fp32 inputs with one degenerate pattern per head: 0 no write (beta or
    both gates 0), 1 no decay (g = 0), 2 a zero key every other step, 3
    near-total forgetting (g = -30) every third step, 4 a zero query, 5 none."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, U, H, d)).astype(np.float32) / np.float32(np.sqrt(d))
    k = rng.standard_normal((T, U, H, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True).astype(np.float32)
    v = rng.standard_normal((T, U, H, d)).astype(np.float32)
    channel = variant != W.GDN
    g = -rng.uniform(0.0, 1.0, (T, U, H, d) if channel else (T, U, H)).astype(np.float32)
    width = 2 * d if variant == W.GDN2 else 1
    beta = None if variant == W.RWKV6 else \
        rng.uniform(0.05, 1.0, (T, U, H, width) if width > 1 else (T, U, H)).astype(np.float32)
    if beta is not None:
        beta[:, :, 0] = 0.0
    g[:, :, 1] = 0.0
    k[1::2, :, 2] = 0.0
    g[::3, :, 3] = -30.0
    q[:, :, 4] = 0.0
    return q, k, v, g, beta


@pytest.mark.parametrize("d,dtype", [(64, "f32"), (128, "bf16")], ids=["d64-f32", "d128-bf16"])
@pytest.mark.parametrize("variant", [W.GDN, W.KDA, W.RWKV6, W.GDN2], ids=["gdn", "kda", "rwkv6", "gated"])
def test_degenerate_inputs_parity(variant, d, dtype):
    """No write, no decay, zero keys, near-total forgetting and zero queries
    reach the oracle's result on every path (log tail left unmerged until the
    final flush)."""
    U, H, T, L = 2, 6, 21, 8
    q, k, v, g, beta = _degenerate_inputs(variant, U, H, d, T)
    # what the kernels read (input dtype) and the same values exactly, for the oracle
    (q_in, q), (k_in, k), (v_in, v) = (W.store(x, dtype) for x in (q, k, v))
    S0 = (0.3 * np.random.default_rng(3).standard_normal((U, H, d, d))).astype(np.float32)
    P = U * H
    o_ref, S_ref = oracle.run(variant, q.reshape(T, P, d), k.reshape(T, P, d), v.reshape(T, P, d),
                              g.reshape((T, P, d) if variant != W.GDN else (T, P)),
                              None if beta is None else beta.reshape((T, P, -1) if variant == W.GDN2 else (T, P)),
                              S0.reshape(P, d, d), np.zeros(P, dtype=np.int64))
    paths = ("eager", "af", "af-fused") if variant == W.GDN2 else \
        ("eager", "log", "log-fused", "af", "af-fused")
    for path in paths:
        st = B.DecodeState(variant, U, H, d, 0 if path == "eager" else L, dtype,
                           merge_on_step=path.endswith("-fused"),
                           log_form=B.DL_LOG_FACTORS if path.startswith("af") else B.DL_LOG_WY)
        st.base.copy_(torch.from_numpy(S0))
        outs = []
        for t in range(T):
            args = tuple(to_torch(x[t], dtype) for x in (q_in, k_in, v_in)) + \
                tuple(None if x is None else torch.from_numpy(np.ascontiguousarray(x[t])).cuda()
                      for x in (g, beta))
            if path == "eager":
                outs.append(st.step_eager(*args))
            else:
                outs.append(st.step_log(*args))
                if (t + 1) % L == 0:
                    st.merge(B.DL_MERGE_FULL)
        if path != "eager":
            st.merge(B.DL_MERGE_ALL)
        assert st.check() == 0
        o = torch.stack(outs, 0).double().cpu().numpy().reshape(T, P, d).transpose(1, 0, 2)
        S = st.base.double().cpu().numpy().reshape(P, d, d)
        eo = per_pair_error(o, o_ref.transpose(1, 0, 2))
        eS = per_pair_error(S, S_ref)
        log(f"  degenerate {variant} {path}: max rel err o {eo.max():.2e}, S {eS.max():.2e}")
        assert eo.max() <= TOL and eS.max() <= TOL, (path, eo, eS)
        # a zero query reads out exactly zero
        assert np.all(o[4::H] == 0.0)
        st.close()
