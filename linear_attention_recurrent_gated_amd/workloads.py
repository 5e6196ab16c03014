"""Seeded synthetic inputs for decode-time gated delta-rule recurrences.

This module draws numbers and stores them in the dtypes the kernels consume.
It holds none of the recurrence's arithmetic: it is the one piece shared by
the HIP path (tests, bench) and the float64 oracle, which both receive the
exact same arrays.

Workloads follow the decode settings the DeltaLog page ("DeltaLog: Deferred
Materialization of Recurrent States for Linear Attention Decoding",
Technical Summary, Problem and Results) describes: a fixed-size
``d_v x d_k`` state per (sequence, layer, head), compact per-token updates
(q, k, v, a decay and a write strength), many sequences decoding at once.
The pages publish no dataset for this kernel, so every input is synthetic.

Recipe (all draws float64 from numpy's PCG64):

* one independent stream per global decode step ``tau``:
  ``SeedSequence([seed, cfg_id, tau])``; the initial state uses
  ``[seed, cfg_id, 2**32 - 1]`` and ragged log offsets ``[seed, cfg_id, 2**32 - 2]``;
* draw order per step: q, k, v (each ``[units, H, d]``), the write-strength
  logit (``[units, H]``, not drawn for the additive variant; ``[units, H,
  d_k + d_v]`` -- erase gate, then write gate -- for the gated form), the decay
  logit (``[units, H]`` for head-wise decay, ``[units, H, d_k]`` for channel-wise);
* q and k are L2-normalised in float64 where the workload says so, then
  rounded to float32 (round-to-nearest-even) and, for bf16 storage, from
  float32 to bf16 (round-to-nearest-even);
* ``beta = sigmoid(x)``; log-decay ``g = -softplus(x)`` (gated delta rule,
  channel-wise KDA decay) or ``g = -exp(x)`` (RWKV6-style decay); both are
  computed in float64 and stored float32.  Kernels and oracle use
  ``alpha = exp(g)``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GDN, KDA, RWKV6, GDN2 = 0, 1, 2, 3
VARIANT_NAMES = {GDN: "gdn", KDA: "kda", RWKV6: "rwkv6", GDN2: "gated"}

_STATE_STREAM = 2**32 - 1
_OFFSET_STREAM = 2**32 - 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input distributions of one synthetic decode workload.

    ``units`` below means state slots handed to one library call: for a
    stacked multi-layer workload each layer is its own state of ``batch``
    units; ``pairs`` are (unit, head) states of ``d_v x d_k`` fp32.
    """

    name: str
    cfg_id: int
    variant: int
    batch: int
    layers: int
    heads: int
    d_k: int
    d_v: int
    steps: int
    log_lens: tuple
    dtype: str                 # storage dtype of q/k/v: "f32" or "bf16"
    qk_l2norm: bool
    state_std: float           # 0.0 -> zero initial state
    decay_mean: float
    decay_std: float
    ragged: bool = False       # per-sequence log fill offsets at start

    @property
    def channel_decay(self) -> bool:
        return self.variant in (KDA, RWKV6, GDN2)

    @property
    def beta_width(self) -> int:
        """Write-strength values per (unit, head): 1, or erase + write gates."""
        return self.d_k + self.d_v if self.variant == GDN2 else 1

    @property
    def has_beta(self) -> bool:
        return self.variant != RWKV6

    @property
    def units_total(self) -> int:
        return self.batch * self.layers

    @property
    def pairs_per_layer(self) -> int:
        return self.batch * self.heads

    def prefix_steps(self, L: int) -> int:
        """Untimed global steps that fill ragged logs before the measured ones."""
        return L - 1 if self.ragged else 0

    def total_steps(self, L: int) -> int:
        return self.prefix_steps(L) + self.steps

    def scaled(self, **kw) -> "Workload":
        """Same distributions, other sizes (for parity cases the oracle finishes fast)."""
        kw.setdefault("name", self.name + "-scaled")
        return dataclasses.replace(self, **kw)


# The decode workloads: a tiny single-head case, four serving shapes (GDN,
# a per-key-decay sweep over L, a ragged multi-layer GDN set and RWKV6) and
# the gated form; the distributions are in the module docstring.
TINY_GDN = Workload("tiny-gdn-d64", 1, GDN, batch=1, layers=1, heads=1, d_k=64, d_v=64,
                    steps=256, log_lens=(8,), dtype="f32", qk_l2norm=True, state_std=0.0,
                    decay_mean=0.0, decay_std=1.0)
GDN_HYBRID = Workload("gdn-b64-h32-d128", 2, GDN, batch=64, layers=1, heads=32, d_k=128,
                      d_v=128, steps=512, log_lens=(16,), dtype="bf16", qk_l2norm=True,
                      state_std=0.02, decay_mean=0.0, decay_std=1.0)
KDA_SWEEP = Workload("kda-b128-h32-d128", 3, KDA, batch=128, layers=1, heads=32, d_k=128,
                     d_v=128, steps=512, log_lens=(1, 4, 8, 16, 32, 64), dtype="bf16",
                     qk_l2norm=True, state_std=0.0, decay_mean=-1.0, decay_std=1.0)
GDN_LARGE = Workload("gdn-b256-l8-h32-d128-ragged", 4, GDN, batch=256, layers=8, heads=32,
                     d_k=128, d_v=128, steps=256, log_lens=(32,), dtype="bf16",
                     qk_l2norm=True, state_std=0.02, decay_mean=0.0, decay_std=1.0,
                     ragged=True)
RWKV6_ADD = Workload("rwkv6-b512-h64-d64", 5, RWKV6, batch=512, layers=1, heads=64, d_k=64,
                     d_v=64, steps=1024, log_lens=(32,), dtype="bf16", qk_l2norm=False,
                     state_std=0.0, decay_mean=-0.5, decay_std=0.5)

# Beyond the five: the gated form (channel-wise erase and write gates) at the
# KDA sweep's shape and decay distribution.
GATED = Workload("gated-b128-h32-d128", 6, GDN2, batch=128, layers=1, heads=32, d_k=128,
                 d_v=128, steps=512, log_lens=(16,), dtype="bf16", qk_l2norm=True,
                 state_std=0.0, decay_mean=-1.0, decay_std=1.0)

WORKLOADS = {w.cfg_id: w for w in (TINY_GDN, GDN_HYBRID, KDA_SWEEP, GDN_LARGE, RWKV6_ADD, GATED)}


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x32)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x64: np.ndarray, dtype: str):
    """Round float64 draws to the storage dtype.

    Returns ``(stored, exact_f32)``: ``stored`` is what the kernels read
    (float32 array, or uint16 bf16 bit patterns), ``exact_f32`` holds the same
    values as float32 (exact for both dtypes) for the oracle.
    """
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == "f32":
        return x32, x32
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class StepInputs:
    """One global decode step for all ``units_total`` units of a workload.

    ``q/k/v``: stored arrays ``[units_total, H, d]`` (float32 or bf16 bits);
    ``*_f32``: the same values as float32; ``g``: float32 ``[units_total, H]``
    or ``[units_total, H, d_k]``; ``beta``: float32 ``[units_total, H]``
    (gated form: ``[units_total, H, d_k + d_v]``) or None.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_f32: np.ndarray
    k_f32: np.ndarray
    v_f32: np.ndarray
    g: np.ndarray
    beta: np.ndarray | None


def _rng(seed: int, cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, stream])))


def draw_step(wl: Workload, tau: int, seed: int = 0) -> StepInputs:
    """Inputs of global step ``tau`` (one independent stream per step)."""
    rng = _rng(seed, wl.cfg_id, tau)
    U, H = wl.units_total, wl.heads
    q = rng.standard_normal((U, H, wl.d_k))
    k = rng.standard_normal((U, H, wl.d_k))
    v = rng.standard_normal((U, H, wl.d_v))
    beta = None
    if wl.variant == GDN2:
        beta = _sigmoid(rng.standard_normal((U, H, wl.d_k + wl.d_v))).astype(np.float32)
    elif wl.has_beta:
        beta = _sigmoid(rng.standard_normal((U, H))).astype(np.float32)
    dshape = (U, H, wl.d_k) if wl.channel_decay else (U, H)
    x = wl.decay_mean + wl.decay_std * rng.standard_normal(dshape)
    g = (-np.exp(x) if wl.variant == RWKV6 else -_softplus(x)).astype(np.float32)
    if wl.qk_l2norm:
        q, k = _l2norm(q), _l2norm(k)
    qs, qf = store(q, wl.dtype)
    ks, kf = store(k, wl.dtype)
    vs, vf = store(v, wl.dtype)
    return StepInputs(qs, ks, vs, qf, kf, vf, g, beta)


def draw_steps(wl: Workload, taus, seed: int = 0, threads: int | None = None):
    """``draw_step`` for many steps, in parallel threads (numpy releases the GIL)."""
    taus = list(taus)
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(taus) <= 1:
        return [draw_step(wl, t, seed) for t in taus]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda t: draw_step(wl, t, seed), taus))


def initial_state(wl: Workload, seed: int = 0) -> np.ndarray:
    """Initial fp32 states ``[units_total, H, d_v, d_k]`` (zeros or N(0, std^2))."""
    shape = (wl.units_total, wl.heads, wl.d_v, wl.d_k)
    if wl.state_std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    rng = _rng(seed, wl.cfg_id, _STATE_STREAM)
    return (wl.state_std * rng.standard_normal(shape)).astype(np.float32)


def ragged_offsets(wl: Workload, L: int, seed: int = 0) -> np.ndarray:
    """Per-sequence log fill offsets ``f_b`` uniform in ``[0, L)`` (zeros if not ragged)."""
    if not wl.ragged:
        return np.zeros(wl.batch, dtype=np.int32)
    rng = _rng(seed, wl.cfg_id, _OFFSET_STREAM)
    return rng.integers(0, L, size=wl.batch).astype(np.int32)


def first_active_step(wl: Workload, L: int, seed: int = 0) -> np.ndarray:
    """Global step at which each sequence starts decoding, ``[batch]``.

    Ragged workloads run an untimed prefix of ``L-1`` global steps in which
    sequence ``b`` joins at ``L-1-f_b``; after the prefix its log holds
    ``f_b`` entries.  Other workloads start every sequence at step 0.
    """
    f = ragged_offsets(wl, L, seed)
    return (wl.prefix_steps(L) - f).astype(np.int32) if wl.ragged else f * 0


def active_rows(wl: Workload, L: int, tau: int, seed: int = 0) -> np.ndarray:
    """Sequences (int32, ascending) that decode at global step ``tau``."""
    return np.nonzero(first_active_step(wl, L, seed) <= tau)[0].astype(np.int32)
