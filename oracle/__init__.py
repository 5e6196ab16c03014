"""Float64 CPU oracle for decode-time gated delta-rule recurrences.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library, and the GPU library never
falls back to it.

* :func:`run` -- the plain step-by-step recurrence in float64 (C, OpenMP over
  independent states; ``recurrence.c``).  It follows the operator list of the
  DeltaLog page (Technical Summary, Kernel Implementation) with the update
  formulas written out in ``recurrence.c``.
* :func:`additive_factor` -- the per-step factor ``a_t`` that an
  additive-factor log stores (numpy, float64).
* :mod:`oracle.exact` -- exact rational (``fractions.Fraction``) models used
  to pin the float64 oracle and the deferred base + log algebra.
* :mod:`oracle.quant` -- a base kept in INT8 with fp32 key channels (a
  reading of the DAMP abstract): the quantiser, its inverse, and the
  recurrence that re-quantises the base at every merge.

Parity status: every function here is pinned by the CPU tests:
:func:`run` and :func:`additive_factor` in ``tests/test_oracle_pins.py``
(brute-force product expansion, the delta-rule write invariant, the identity
case, closed forms and the exact equality of eager and deferred schedules),
:func:`readout` in ``tests/test_oracle_readout.py`` (the recurrence's own last
output and a hand-worked example, with planted mistakes that must fail),
:mod:`oracle.quant` in ``tests/test_oracle_quant.py`` (grid values, ties to
even, the rounding error bound, zero rows and kept outliers, planted
quantiser mistakes; the mixed recurrence against the plain one and against
the deferred log's schedule model).  The pages print no worked numeric
example, so no stored value comes from them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build_oracle, needs_build

GDN, KDA, RWKV6, GDN2 = 0, 1, 2, 3

_libs: dict = {}


def _load(path: str | None = None):
    """Load the oracle library (``path`` overrides it, e.g. for mutation tests)."""
    key = path or LIB_PATH
    if key not in _libs:
        if path is None and needs_build():
            build_oracle()
        lib = ctypes.CDLL(key)
        lib.oracle_run.restype = ctypes.c_int
        lib.oracle_run.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_run_f64_state.restype = ctypes.c_int
        lib.oracle_run_f64_state.argtypes = lib.oracle_run.argtypes
        lib.oracle_max_threads.restype = ctypes.c_int
        _libs[key] = lib
    return _libs[key]


def affinity_cores() -> int:
    """Cores in this process's affinity mask."""
    return len(os.sched_getaffinity(0))


def default_threads() -> int:
    """Every core in this process's affinity mask, capped by ``OMP_NUM_THREADS``
    when that is set (a host that shares its cores sets it to this process's
    share)."""
    n = affinity_cores()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def run(variant: int, q, k, v, g, beta=None, S0=None, t_start=None, threads: int | None = None,
        lib_path: str | None = None, S0_f64=None):
    """Run the recurrence for ``P`` independent states over ``T`` steps.

    Shapes: ``q, k`` ``[T, P, d_k]``; ``v`` ``[T, P, d_v]``; ``g`` ``[T, P]``
    (head-wise decay) or ``[T, P, d_k]`` (channel-wise); ``beta`` ``[T, P]``
    (not used by the additive variant; ``[T, P, d_k + d_v]`` -- erase gate,
    then write gate -- for the gated form); ``S0`` ``[P, d_v, d_k]`` or None for
    zeros; ``t_start`` ``[P]`` first step each state takes (outputs before it
    are zero).  All float inputs are the exact values the kernels consume.
    ``S0_f64`` ``[P, d_v, d_k]`` float64 replaces ``S0`` when the initial state
    is not an fp32 value (a dequantised base).

    Returns ``(o, S)``: float64 ``[T, P, d_v]`` and ``[P, d_v, d_k]``.
    """
    q, k, v, g, beta, S0 = (_f32(x) for x in (q, k, v, g, beta, S0))
    T, P, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, P, dk) and v.shape == (T, P, dv)
    if variant == GDN:
        assert g.shape == (T, P)
    else:
        assert g.shape == (T, P, dk)
    if variant == GDN2:
        assert beta is not None and beta.shape == (T, P, dk + dv)
    elif variant != RWKV6:
        assert beta is not None and beta.shape == (T, P)
    else:
        beta = None
    if S0 is not None:
        assert S0.shape == (P, dv, dk)
    ts = None
    if t_start is not None:
        ts = np.ascontiguousarray(t_start, dtype=np.int32)
        assert ts.shape == (P,)
    o = np.zeros((T, P, dv), dtype=np.float64)
    S = np.zeros((P, dv, dk), dtype=np.float64)
    lib = _load(lib_path)
    if S0_f64 is not None:
        S0d = np.ascontiguousarray(S0_f64, dtype=np.float64)
        assert S0d.shape == (P, dv, dk)
        rc = lib.oracle_run_f64_state(variant, P, dk, dv, T, _ptr(S0d), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), _ptr(beta), _ptr(ts), _ptr(o), _ptr(S),
                                      int(threads or default_threads()))
    else:
        rc = lib.oracle_run(variant, P, dk, dv, T, _ptr(S0), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(g), _ptr(beta), _ptr(ts), _ptr(o), _ptr(S),
                            int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_run failed with code {rc}")
    return o, S


def readout(S, q):
    """``o = S q`` for states ``[P, d_v, d_k]`` and queries ``[P, d_k]`` (float64)."""
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return np.einsum("pij,pj->pi", S, q)


def additive_factor(variant: int, S_prev, k, v, g, beta=None):
    """The compact update factor ``a_t`` of one step, in float64.

    A step writes ``S_t = S_{t-1} diag(alpha_t) + a_t k_t^T`` with
    ``alpha_t = exp(g_t)`` (a scalar for the head-wise decay) and
    ``a_t = beta_t (v_t - S_{t-1} (alpha_t * k_t))`` for the delta-rule
    operators, ``a_t = w_t * v_t - S_{t-1} (alpha_t * e_t * k_t)`` for the
    gated form (erase gate ``e_t``, write gate ``w_t``), ``a_t = v_t`` for the
    additive one: the factor pair ``(a_t, b_t = k_t)`` that the DeltaLog
    page's Core Mechanism appends to the log instead of writing the state.

    Shapes: ``S_prev`` ``[P, d_v, d_k]``; ``k`` ``[P, d_k]``; ``v`` ``[P, d_v]``;
    ``g`` ``[P]`` or ``[P, d_k]``; ``beta`` ``[P]`` (gated: ``[P, d_k + d_v]``).
    Returns ``[P, d_v]``.
    """
    S = np.asarray(S_prev, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if variant == RWKV6:
        return v.copy()
    g = np.asarray(g, dtype=np.float64)
    alpha = np.exp(g)[:, None] if variant == GDN else np.exp(g)
    beta = np.asarray(beta, dtype=np.float64)
    if variant == GDN2:
        dk = k.shape[1]
        erase, write = beta[:, :dk], beta[:, dk:]
        return write * v - np.einsum("pij,pj->pi", S, alpha * erase * k)
    x = np.einsum("pij,pj->pi", S, alpha * k)
    return beta[:, None] * (v - x)


def max_threads() -> int:
    return int(_load().oracle_max_threads())
