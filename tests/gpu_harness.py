"""Runs a decode workload through the GPU library and the float64 oracle on
the same seeded inputs, and compares them.

Every input step is drawn once; the GPU consumes the whole batch, the oracle
the selected (unit, head) pairs.  The GPU paths run side by side (each with
its own state block) in one step loop.
"""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import bench
import oracle
from linear_attention_recurrent_gated_amd import binding as B
from linear_attention_recurrent_gated_amd import workloads as W

TOL = 2e-4


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def log(msg):
    print(msg, flush=True)


class Case:
    """Outputs of one run: per path, ``o`` [n_sel, T, d] and final ``S`` [n_sel, d, d]."""

    def __init__(self):
        self.gpu = {}
        self.ref = None
        self.fills = []


def run_case(wl: W.Workload, L: int, paths=("eager", "log"), seed: int = 0,
             steps: int | None = None, pairs=None, merge_every_step: bool | None = None,
             run_oracle: bool = True, threads: int | None = None, on_step=None,
             bench_schedule: bool = False) -> Case:
    """Run ``paths`` (subset of "eager", "log", "log-replay", "log-fused",
    "af", "af-fused") over the workload.

    "log" merges a full log with the WY merge after the step that fills it,
    "log-replay" with the replay merge, "log-fused" inside that step; "af"
    and "af-fused" are the same two schedules with the additive-factor log.

    ``pairs``: selected flat pair indices (unit_total * H + head) to record;
    None records all.  ``on_step(tau, states)`` is called after each step.
    ``bench_schedule``: launch what the benchmark launches for ragged logs --
    separate merges name only the units whose logs are full (``slot_idx``),
    and a step that merges in place takes its rows in the benchmark's order
    (``row_order``) -- instead of a merge over every unit after each step;
    with several layers, a path with separate merges keeps every layer's
    states in one block and merges once per step, after the last layer, over
    every layer's full logs, as the benchmark does.
    """
    H, d, Bt, layers = wl.heads, wl.d_k, wl.batch, wl.layers
    T = wl.total_steps(L) if steps is None else steps
    P = wl.units_total * H
    sel = np.arange(P) if pairs is None else np.asarray(pairs)
    sel_u, sel_h = sel // H, sel % H
    first = W.first_active_step(wl, L, seed)                     # [batch]
    first_u = np.tile(first, layers)                             # [units_total]
    if merge_every_step is None:
        merge_every_step = wl.ragged and not bench_schedule
    fills = np.zeros(Bt, dtype=np.int64)                         # host model of the schedule

    S0 = W.initial_state(wl, seed)                               # [U, H, d, d]
    def pooled(path):
        return bench_schedule and wl.ragged and layers > 1 and path in ("log", "log-replay", "af")

    sblocks, states = {}, {}
    for path in paths:
        nblk, ublk = (1, layers * Bt) if pooled(path) else (layers, Bt)
        sblocks[path] = []
        for l in range(nblk):
            st = B.DecodeState(wl.variant, ublk, H, d, 0 if path == "eager" else L, wl.dtype,
                               merge_on_step=path.endswith("-fused"),
                               log_form=B.DL_LOG_FACTORS if path.startswith("af") else B.DL_LOG_WY)
            st.base.copy_(torch.from_numpy(S0[l * ublk:(l + 1) * ublk]))
            sblocks[path].append(st)
        states[path] = [sblocks[path][0 if pooled(path) else l] for l in range(layers)]
    torch.cuda.synchronize()

    rec = {path: [] for path in paths}
    q_sel, k_sel, v_sel, g_sel, b_sel = [], [], [], [], []
    sel_u_t = torch.from_numpy(sel_u).cuda()
    sel_h_t = torch.from_numpy(sel_h).cuda()

    taus = list(range(T))
    pool = ThreadPoolExecutor(max_workers=1)
    nthreads = threads or min(16, len(__import__("os").sched_getaffinity(0)))
    chunk = 16

    def draw(block):
        return W.draw_steps(wl, block, seed, threads=nthreads)

    blocks = [taus[i:i + chunk] for i in range(0, T, chunk)]
    fut = pool.submit(draw, blocks[0]) if blocks else None
    t0 = time.time()
    for bi, block in enumerate(blocks):
        drawn = fut.result()
        if bi + 1 < len(blocks):
            fut = pool.submit(draw, blocks[bi + 1])
        for tau, s in zip(block, drawn):
            q = to_torch(s.q, wl.dtype)
            k = to_torch(s.k, wl.dtype)
            v = to_torch(s.v, wl.dtype)
            g = torch.from_numpy(s.g).cuda()
            beta = None if s.beta is None else torch.from_numpy(s.beta).cuda()
            if run_oracle:
                q_sel.append(s.q_f32.reshape(P, -1)[sel])
                k_sel.append(s.k_f32.reshape(P, -1)[sel])
                v_sel.append(s.v_f32.reshape(P, -1)[sel])
                g_sel.append(s.g.reshape(P, -1)[sel] if wl.channel_decay else s.g.reshape(P)[sel])
                if s.beta is not None:
                    b_sel.append(s.beta.reshape((P,) if wl.beta_width == 1 else (P, -1))[sel])
            act = np.nonzero(first <= tau)[0]
            # units whose logs this step fills (the benchmark's host model)
            full_next = np.nonzero(fills + np.isin(np.arange(Bt), act) == L)[0]
            for path in paths:
                o_full = torch.zeros((wl.units_total, H, d), dtype=torch.float32, device="cuda")
                order = None
                if bench_schedule and path.endswith("-fused") and len(act) == Bt:
                    o_np = bench.row_order("auto", fills, L)
                    if o_np is not None:
                        order = torch.from_numpy(o_np.astype(np.int32)).cuda()
                for l in range(layers):
                    st = states[path][l]
                    lo, hi = l * Bt, (l + 1) * Bt
                    if len(act) == 0:
                        continue
                    if len(act) == Bt:
                        idx, slot = None, None
                        args = (q[lo:hi], k[lo:hi], v[lo:hi], g[lo:hi],
                                None if beta is None else beta[lo:hi])
                    else:
                        idx = torch.from_numpy(act.astype(np.int64)).cuda()
                        slot = torch.from_numpy(act.astype(np.int32)).cuda()
                        args = tuple(None if x is None else x[lo:hi].index_select(0, idx).contiguous()
                                     for x in (q, k, v, g, beta))
                    if pooled(path):                  # layer l's units in the shared block
                        slot = torch.from_numpy((l * Bt + act).astype(np.int32)).cuda()
                    if path == "eager":
                        o = st.step_eager(*args, slot_idx=slot)
                    else:
                        o = st.step_log(*args, slot_idx=slot, row_order=order)
                        if bench_schedule and wl.ragged:
                            if pooled(path) and len(full_next) and l == layers - 1:
                                ms = np.concatenate([j * Bt + full_next for j in range(layers)])
                                st.merge(B.DL_MERGE_FULL, slot_idx=torch.from_numpy(ms.astype(np.int32)).cuda(),
                                         replay=(path == "log-replay"))
                            elif not pooled(path) and not path.endswith("-fused") and len(full_next):
                                st.merge(B.DL_MERGE_FULL, slot_idx=torch.from_numpy(
                                    full_next.astype(np.int32)).cuda(), replay=(path == "log-replay"))
                        elif merge_every_step or (tau + 1) % L == 0:
                            st.merge(B.DL_MERGE_FULL, replay=(path == "log-replay"))
                    if idx is None:
                        o_full[lo:hi] = o
                    else:
                        o_full[lo:hi].index_copy_(0, idx, o)
                rec[path].append(o_full[sel_u_t, sel_h_t])
            fills[act] += 1
            fills[fills == L] = 0
            if on_step is not None:
                on_step(tau, states)
        if bi % 8 == 0:
            log(f"  [{wl.name} L={L}] steps {block[0]}..{block[-1]} done ({time.time() - t0:.1f}s)")
    pool.shutdown()

    case = Case()
    for path in paths:
        finals = []
        for st in sblocks[path]:
            if path != "eager":
                st.merge(B.DL_MERGE_ALL, replay=(path == "log-replay"))
            finals.append(st.base)
        flags = [st.check() for st in sblocks[path]]
        assert not any(flags), f"device flags {flags} on path {path}"
        Sfull = torch.cat(finals, 0)                              # [U, H, d, d]
        S_sel = Sfull[sel_u_t, sel_h_t].double().cpu().numpy()
        o_sel = torch.stack(rec[path], 1).double().cpu().numpy()  # [n_sel, T, d]
        case.gpu[path] = (o_sel, S_sel)
        for st in sblocks[path]:
            st.close()
    if run_oracle:
        beta_arr = np.stack(b_sel) if b_sel else None
        S0_sel = S0.reshape(P, d, d)[sel]
        t_start = first_u[sel_u]
        o_ref, S_ref = oracle.run(wl.variant, np.stack(q_sel), np.stack(k_sel), np.stack(v_sel),
                                  np.stack(g_sel), beta_arr, S0_sel, t_start)
        case.ref = (o_ref.transpose(1, 0, 2), S_ref)
    return case


def per_pair_error(gpu: np.ndarray, ref: np.ndarray):
    """max |gpu - ref| / max(1, max |ref|) per pair (axis 0)."""
    n = gpu.shape[0]
    diff = np.abs(gpu - ref).reshape(n, -1).max(axis=1)
    scale = np.maximum(1.0, np.abs(ref).reshape(n, -1).max(axis=1))
    return diff / scale


def assert_parity(case: Case, tol: float = TOL, label: str = ""):
    o_ref, S_ref = case.ref
    for path, (o, S) in case.gpu.items():
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)), f"{label} {path}: non-finite"
        eo = per_pair_error(o, o_ref)
        eS = per_pair_error(S, S_ref)
        log(f"  {label} {path}: max rel err o {eo.max():.2e}, S {eS.max():.2e}")
        assert eo.max() <= tol, f"{label} {path}: outputs off by {eo.max():.3e} (pair {eo.argmax()})"
        assert eS.max() <= tol, f"{label} {path}: final state off by {eS.max():.3e} (pair {eS.argmax()})"
