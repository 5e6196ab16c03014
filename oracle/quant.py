"""Mixed-precision base of a deferred recurrent state: INT8 codes with fp32
key channels (float64 oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Shares no code with
the GPU library.

The DAMP abstract ("DAMP: Decay-Aware Mixed-Precision Recurrent-State
Quantization", on the Jianchao Tan author page) stores most of a recurrent
state in INT8 and a small set of channels, chosen offline, at higher
precision.  It leaves the INT8 scale granularity and the kept channels'
format open; these functions take the plainest reading:

* the kept channels are key channels (columns of the ``d_v x d_k`` state),
  one set per head, given as column indices, and keep their fp32 values;
* every other entry is a symmetric INT8 code with one fp32 scale per value
  row: ``amax_i = max_j |S_ij|`` over the other columns,
  ``scale_i = amax_i / 127``, ``code_ij = clip(rint(S_ij / scale_i), -127,
  127)`` (fp32 divisions, ties to even), all codes 0 when ``scale_i`` is 0;
  the kept columns' codes are 0;
* the dequantised base is ``code_ij * scale_i`` (exact in float64) and the
  kept values;
* with a deferred log the base is quantised when a state is imported and
  again, from the fp32 state, at every merge; between merges the state
  evolves as the plain recurrence does from the dequantised base (the log
  keeps exact factors).  The DeltaLog page's Core Mechanism (a read-only
  base, a bounded log, a periodic merge) fixes when merges happen.
"""
from __future__ import annotations

import numpy as np

QMAX = 127


def _mask(dk: int, hp_idx) -> np.ndarray:
    """[P, dk] bool: the kept key channels of each state."""
    hp_idx = np.asarray(hp_idx, dtype=np.int64)
    m = np.zeros((hp_idx.shape[0], dk), dtype=bool)
    for p in range(hp_idx.shape[0]):
        m[p, hp_idx[p]] = True
    return m


def quantize_base(X, hp_idx):
    """Quantise fp32 states ``X`` [P, d_v, d_k] with kept columns ``hp_idx``
    [P, M] (per state).  Every decision is taken in float32, as the reading
    above states.  Returns ``(codes int8 [P, d_v, d_k], scale float32 [P,
    d_v], hp float32 [P, d_v, M])``."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    P, dv, dk = X.shape
    hp_idx = np.asarray(hp_idx, dtype=np.int64).reshape(P, -1)
    keep = _mask(dk, hp_idx)[:, None, :]                       # [P, 1, dk]
    mag = np.where(keep, np.float32(0), np.abs(X))
    amax = mag.max(axis=2)                                     # [P, dv], exact
    scale = (amax / np.float32(QMAX)).astype(np.float32)       # IEEE fp32 division
    safe = np.where(scale > 0, scale, np.float32(1))
    ratio = (X / safe[:, :, None]).astype(np.float32)          # IEEE fp32 division
    codes = np.clip(np.rint(ratio), -QMAX, QMAX)               # ties to even
    codes = np.where((scale[:, :, None] > 0) & ~keep, codes, 0).astype(np.int8)
    hp = np.take_along_axis(X, np.broadcast_to(hp_idx[:, None, :], (P, dv, hp_idx.shape[1])), axis=2)
    return codes, scale, np.ascontiguousarray(hp, dtype=np.float32)


def dequantize_base(codes, scale, hp, hp_idx):
    """The states a quantised base stands for, float64 [P, d_v, d_k]."""
    codes = np.asarray(codes)
    P, dv, dk = codes.shape
    hp_idx = np.asarray(hp_idx, dtype=np.int64).reshape(P, -1)
    S = codes.astype(np.float64) * np.asarray(scale, dtype=np.float64)[:, :, None]
    for p in range(P):
        S[p][:, hp_idx[p]] = np.asarray(hp[p], dtype=np.float64)
    return S


def boundary_elements(X, scale, band: float = 1e-3):
    """Entries whose ``X / scale`` lies within ``band`` of a rounding boundary
    (a half-integer): there an fp32 state computed in another order may take
    the neighbouring code.  ``X`` float64 [P, d_v, d_k], ``scale`` [P, d_v]."""
    s = np.asarray(scale, dtype=np.float64)[:, :, None]
    r = np.asarray(X, dtype=np.float64) / np.where(s > 0, s, 1.0)
    frac = np.abs(r - np.floor(r) - 0.5)
    return (frac < band) & (s > 0)


def run_quantized_base(variant, q, k, v, g, beta, S0, t_start, L, hp_idx, threads=None,
                       run=None):
    """The recurrence over a deferred state whose base is kept quantised.

    Inputs as for :func:`oracle.run` (``q, k, v`` [T, P, d]; ``g``, ``beta``
    per step; ``S0`` [P, d_v, d_k] or None; ``t_start`` [P] or None), plus the
    log length ``L`` and the kept columns ``hp_idx`` [P, M].  State ``p`` is
    imported (quantised) before its first step; its log fills one entry per
    step from that step on, and after every ``L``-th of its steps the log
    merges: the float64 state is rounded to fp32 and quantised again.

    Returns ``(o, S, final)``: outputs float64 [T, P, d_v] (zero before a
    state's first step), the float64 logical state after the last step, and
    the quantised base ``(codes, scale, hp)`` after a final flush (the last
    merge's base when the log is empty at the end).
    """
    if run is None:
        from . import run as run          # the plain float64 recurrence
    q = np.asarray(q, dtype=np.float32)
    T, P, dk = q.shape
    dv = np.asarray(v).shape[2]
    hp_idx = np.asarray(hp_idx, dtype=np.int64).reshape(P, -1)
    S0 = np.zeros((P, dv, dk), np.float32) if S0 is None else np.asarray(S0, np.float32)
    ts = np.zeros(P, dtype=np.int64) if t_start is None else np.asarray(t_start, dtype=np.int64)
    o = np.zeros((T, P, dv), dtype=np.float64)
    S_end = np.zeros((P, dv, dk), dtype=np.float64)
    fc = np.zeros((P, dv, dk), dtype=np.int8)
    fs = np.zeros((P, dv), dtype=np.float32)
    fh = np.zeros((P, dv, hp_idx.shape[1]), dtype=np.float32)
    for p in range(P):
        sel = slice(p, p + 1)
        base = quantize_base(S0[sel], hp_idx[sel])
        t = int(ts[p])
        fill = 0
        S = dequantize_base(*base, hp_idx[sel])
        while t < T:
            n = min(L - fill, T - t)
            seg = slice(t, t + n)
            os_, S = run(variant, q[seg][:, sel], np.asarray(k)[seg][:, sel],
                         np.asarray(v)[seg][:, sel], np.asarray(g)[seg][:, sel],
                         None if beta is None else np.asarray(beta)[seg][:, sel],
                         threads=threads or 1, S0_f64=S)
            o[seg, p] = os_[:, 0]
            t += n
            fill += n
            if fill == L:
                base = quantize_base(S.astype(np.float32), hp_idx[sel])
                S = dequantize_base(*base, hp_idx[sel])
                fill = 0
        S_end[p] = S[0]
        if fill > 0:
            base = quantize_base(S.astype(np.float32), hp_idx[sel])
        fc[p], fs[p], fh[p] = base[0][0], base[1][0], base[2][0]
    return o, S_end, (fc, fs, fh)
