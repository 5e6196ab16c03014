"""Exact rational models of the recurrences and of the deferred schedule.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything here works
on ``fractions.Fraction`` values in plain Python lists, for tiny sizes only
(``d <= 8``, ``T <= 16``).  Decays enter as ``alpha`` itself (a positive
rational), so every result is exact.

Notation: a state ``S`` is a ``d_v x d_k`` list of rows; vectors are lists.
Variants: 0 = Gated DeltaNet (scalar ``alpha``), 1 = KDA (per-key-channel
``alpha``), 2 = RWKV6-style additive (per-channel ``w``, no ``beta``),
3 = the gated form (per-key ``alpha``; ``beta`` is a pair ``(e, w)`` of an
erase gate on the key channels and a write gate on the value channels).

Sources:

* the step formulas are the ones written in ``recurrence.c``; the
  DeltaLog page ("DeltaLog: Deferred Materialization of Recurrent States for
  Linear Attention Decoding", Technical Summary, Kernel Implementation)
  names the three operators and their decay granularity;
* the deferred schedule -- a read-only dense base, a bounded log of compact
  per-token updates appended every step, a periodic merge that materialises
  base plus log and resets the log -- is the DeltaLog page's Core Mechanism;
  its claim that this only changes the physical schedule, not the
  recurrence (Methodology), is what :func:`deferred_run` is tested against;
* the additive-factor log (``af_*``) stores the compact factors
  ``(a_t, b_t)`` and the decay snapshot that the Core Mechanism names, with
  ``a_t`` the delta-rule write ``beta_t (v_t - S_{t-1}(alpha_t * k_t))``;
* the merge is written in WY/UT form: a product of rank-one delta-rule
  transforms folded into one triangular solve, the block form the CARVE page
  (abstract) and its Gated DeltaNet-2 neighbour (chunkwise WY algorithm)
  refer to.
"""
from __future__ import annotations

from fractions import Fraction as Fr

GDN, KDA, RWKV6, GDN2 = 0, 1, 2, 3


# ----------------------------------------------------------------------------
# small exact linear algebra
# ----------------------------------------------------------------------------
def zeros(r, c):
    return [[Fr(0)] * c for _ in range(r)]


def eye(n):
    return [[Fr(int(i == j)) for j in range(n)] for i in range(n)]


def matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    assert all(len(row) == m for row in A)
    return [[sum((A[i][t] * B[t][j] for t in range(m)), Fr(0)) for j in range(p)]
            for i in range(n)]


def matvec(A, x):
    return [sum((a * b for a, b in zip(row, x)), Fr(0)) for row in A]


def dot(a, b):
    return sum((x * y for x, y in zip(a, b)), Fr(0))


def outer(a, b):
    return [[x * y for y in b] for x in a]


def madd(A, B, c=Fr(1)):
    return [[x + c * y for x, y in zip(ra, rb)] for ra, rb in zip(A, B)]


def diag(v):
    n = len(v)
    return [[v[i] if i == j else Fr(0) for j in range(n)] for i in range(n)]


def _chan(variant, alpha, dk):
    """Per-key-channel decay vector (a scalar decay is repeated)."""
    if variant == GDN:
        return [Fr(alpha)] * dk
    assert len(alpha) == dk
    return [Fr(a) for a in alpha]


# ----------------------------------------------------------------------------
# eager recurrence
# ----------------------------------------------------------------------------
def transform(variant, alpha, beta, k):
    """The right factor ``A_t`` acting on the old state.

    GDN ``alpha (I - beta k k^T)``; KDA ``diag(alpha) (I - beta k k^T)``;
    RWKV6 ``diag(w)``; gated ``diag(alpha) (I - (e * k) k^T)``.
    """
    dk = len(k)
    D = diag(_chan(variant, alpha, dk))
    if variant == RWKV6:
        return D
    if variant == GDN2:
        e = [Fr(x) * Fr(kk) for x, kk in zip(beta[0], k)]
        return matmul(D, madd(eye(dk), outer(e, k), -Fr(1)))
    return matmul(D, madd(eye(dk), outer(k, k), -Fr(beta)))


def write_term(variant, beta, k, v):
    """The additive term: ``beta v k^T`` (RWKV6: ``v k^T``; gated: ``(w * v) k^T``)."""
    if variant == GDN2:
        return outer([Fr(w) * Fr(x) for w, x in zip(beta[1], v)], k)
    c = Fr(1) if variant == RWKV6 else Fr(beta)
    return [[c * x for x in row] for row in outer(v, k)]


def step(variant, S, q, k, v, alpha, beta):
    """``S_t = S_{t-1} A_t + write``; returns ``(S_t, o_t = S_t q_t)``."""
    S1 = madd(matmul(S, transform(variant, alpha, beta, k)), write_term(variant, beta, k, v))
    return S1, matvec(S1, q)


def run_stepwise(variant, S0, qs, ks, vs, alphas, betas):
    """Step-by-step exact recurrence; returns ``(outputs, final state)``."""
    S = [list(r) for r in S0]
    outs = []
    for t in range(len(ks)):
        b = None if betas is None else betas[t]
        S, o = step(variant, S, qs[t], ks[t], vs[t], alphas[t], b)
        outs.append(o)
    return outs, S


def run_product_expansion(variant, S0, ks, vs, alphas, betas):
    """Brute force: ``S_T = S_0 A_1...A_T + sum_j write_j A_{j+1}...A_T``.

    Every transform is built as an explicit matrix and multiplied out; no
    step reuses a previous state.
    """
    T = len(ks)
    dk = len(ks[0])
    A = [transform(variant, alphas[t], None if betas is None else betas[t], ks[t])
         for t in range(T)]

    def prod(a, b):  # A_a ... A_{b-1} (0-based, identity when empty)
        P = eye(dk)
        for t in range(a, b):
            P = matmul(P, A[t])
        return P

    S = matmul(S0, prod(0, T))
    for j in range(T):
        w = write_term(variant, None if betas is None else betas[j], ks[j], vs[j])
        S = madd(S, matmul(w, prod(j + 1, T)))
    return S


# ----------------------------------------------------------------------------
# deferred (base + log) schedule
# ----------------------------------------------------------------------------
def qchain_readout(variant, base, log, q):
    """Readout of base + log without materialising the state.

    Pulls ``q`` back through the logged transforms, newest first:
    ``coef_j = beta_j k_j . q_j`` (RWKV6: ``k_j . q_j``) and
    ``q_{j-1} = alpha_j * (q_j - coef_j k_j)`` (RWKV6: ``w_j * q_j``); then
    ``o = base q_0 + sum_j coef_j v_j``.  ``log`` holds
    ``(k, v, alpha, beta)`` tuples, oldest first.
    """
    dk = len(q)
    qq = [Fr(x) for x in q]
    coef = [Fr(0)] * len(log)
    for j in range(len(log) - 1, -1, -1):
        k, v, alpha, beta = log[j]
        a = _chan(variant, alpha, dk)
        if variant == RWKV6:
            coef[j] = dot(k, qq)
            qq = [ai * x for ai, x in zip(a, qq)]
        else:
            coef[j] = Fr(beta) * dot(k, qq)
            qq = [ai * (x - coef[j] * kk) for ai, x, kk in zip(a, qq, k)]
    o = matvec(base, qq)
    for j, (k, v, alpha, beta) in enumerate(log):
        o = [x + coef[j] * vv for x, vv in zip(o, v)]
    return o


def wy_t_column(variant, log, j):
    """Coupling column ``N[:j, j]`` of logged entry j (0-based) to the earlier ones.

    ``N_ij = beta_i sum_c k_i[c] k_j[c] D(i, j)[c]`` for ``i < j``: entry i's
    coefficient depends on entry j's through it.  Appending entry j adds one
    column to ``R = (I + N)^{-1}``: ``R[:j, j] = -R[:j, :j] N[:j, j]``,
    ``R[j, j] = 1`` (see :func:`wy_build_r`).  The additive variant has no
    coupling (``R = I``).
    """
    dk = len(log[0][0])
    decays = [_chan(variant, e[2], dk) for e in log]

    def D(i, jj):
        out = [Fr(1)] * dk
        for m in range(i + 1, jj + 1):
            out = [x * y for x, y in zip(out, decays[m])]
        return out

    if variant == RWKV6:
        return [Fr(0)] * j + [Fr(1)]
    kj = [Fr(x) for x in log[j][0]]
    u = []
    for i in range(j):
        ki = [Fr(x) for x in log[i][0]]
        u.append(Fr(log[i][3]) * sum((a * b * c for a, b, c in zip(ki, kj, D(i, j))), Fr(0)))
    return u


def wy_build_r(variant, log):
    """R = (I + N)^{-1} (upper triangular, unit diagonal) built one column per entry."""
    n = len(log)
    R = [[Fr(int(i == j)) for j in range(n)] for i in range(n)]
    for j in range(1, n):
        u = wy_t_column(variant, log, j)
        if variant == RWKV6:
            continue
        for i in range(j):
            R[i][j] = -sum((R[i][m] * u[m] for m in range(i, j)), Fr(0))
    return R


def wy_readout(variant, base, log, q):
    """Readout of base + log in compact WY form, with no sequential chain.

    With ``E_j`` the decay accumulated over entries ``0..j`` and
    ``D(j, c)`` the decay of entries ``j+1..c`` (c the newest):
    ``r_j = beta_j k_j . (D(j, c) * q)`` (additive: beta = 1),
    ``coef = R r``, ``q0 = E_c * q - sum_j coef_j E_j * k_j`` (additive: no
    k terms, ``coef = r``), and ``o = base q0 + sum_j coef_j v_j``.
    """
    n = len(log)
    dk = len(q)
    if n == 0:
        return matvec(base, [Fr(x) for x in q])
    decays = [_chan(variant, e[2], dk) for e in log]
    E = []
    acc = [Fr(1)] * dk
    for a in decays:
        acc = [x * y for x, y in zip(acc, a)]
        E.append(acc)
    c = n - 1

    def D(j, i):
        out = [Fr(1)] * dk
        for m in range(j + 1, i + 1):
            out = [x * y for x, y in zip(out, decays[m])]
        return out

    qf = [Fr(x) for x in q]
    r = []
    for j, (k, v, alpha, beta) in enumerate(log):
        b = Fr(1) if variant == RWKV6 else Fr(beta)
        r.append(b * sum((Fr(kk) * d * x for kk, d, x in zip(k, D(j, c), qf)), Fr(0)))
    if variant == RWKV6:
        coef = r
        q0 = [e * x for e, x in zip(E[c], qf)]
    else:
        R = wy_build_r(variant, log)
        coef = [sum((R[i][j] * r[j] for j in range(i, n)), Fr(0)) for i in range(n)]
        q0 = [e * x for e, x in zip(E[c], qf)]
        for j, (k, v, alpha, beta) in enumerate(log):
            q0 = [x - coef[j] * ej * Fr(kk) for x, ej, kk in zip(q0, E[j], k)]
    o = matvec(base, q0)
    for j, (k, v, alpha, beta) in enumerate(log):
        o = [x + coef[j] * Fr(vv) for x, vv in zip(o, v)]
    return o


def wy_solve_u(variant, base, log):
    """Columns ``U_j`` of the WY merge's triangular solve (see :func:`wy_merge`).

    ``W_j = base (k_j * P_j)``, ``M_ij = beta_j sum_c k_i[c] k_j[c] D(i, j)[c]``
    (``i < j``), and ``U (I + M) = (V - W) diag(beta)`` by forward
    substitution over columns; RWKV6: ``U = V``.
    """
    n = len(log)
    dk = len(log[0][0])
    decays = [_chan(variant, e[2], dk) for e in log]
    P = []
    acc = [Fr(1)] * dk
    for a in decays:
        acc = [x * y for x, y in zip(acc, a)]
        P.append(acc)

    def D(i, j):  # product of decays of entries i+1..j
        out = [Fr(1)] * dk
        for m in range(i + 1, j + 1):
            out = [x * y for x, y in zip(out, decays[m])]
        return out

    ks = [[Fr(x) for x in e[0]] for e in log]
    vs = [[Fr(x) for x in e[1]] for e in log]
    if variant == RWKV6:
        return vs
    betas = [Fr(e[3]) for e in log]
    W = [matvec(base, [kk * p for kk, p in zip(ks[j], P[j])]) for j in range(n)]
    M = [[Fr(0)] * n for _ in range(n)]
    for i in range(n):
        for j in range(i + 1, n):
            dij = D(i, j)
            M[i][j] = betas[j] * sum((a * b * c for a, b, c in zip(ks[i], ks[j], dij)), Fr(0))
    B = [[betas[j] * (vv - ww) for vv, ww in zip(vs[j], W[j])] for j in range(n)]
    U = []
    for j in range(n):
        col = list(B[j])
        for i in range(j):
            col = [c - u * M[i][j] for c, u in zip(col, U[i])]
        U.append(col)
    return U


def wy_merge(variant, base, log):
    """Materialise ``base`` followed by the logged updates in WY/UT form.

    With ``P_j`` the decay accumulated over entries ``1..j`` and
    ``D(i, j) = P_j / P_i`` (products of the logged decays):

    * ``W_j = base (k_j * P_j)``;
    * ``M_ij = beta_j sum_c k_i[c] k_j[c] D(i, j)[c]`` for ``i < j``;
    * ``U`` solves ``U (I + M) = (V - W) diag(beta)`` (forward substitution
      over columns);
    * ``S' = base diag(P_n) + sum_j U_j (k_j * D(j, n))^T``.

    RWKV6 has no delta correction: ``U = V``.
    """
    n = len(log)
    if n == 0:
        return [list(r) for r in base]
    dk = len(log[0][0])
    decays = [_chan(variant, e[2], dk) for e in log]
    P = []
    acc = [Fr(1)] * dk
    for a in decays:
        acc = [x * y for x, y in zip(acc, a)]
        P.append(acc)

    def D(i, j):  # product of decays of entries i+1..j
        out = [Fr(1)] * dk
        for m in range(i + 1, j + 1):
            out = [x * y for x, y in zip(out, decays[m])]
        return out

    ks = [[Fr(x) for x in e[0]] for e in log]
    U = wy_solve_u(variant, base, log)
    last = n - 1
    S = [[x * p for x, p in zip(row, P[last])] for row in base]
    for j in range(n):
        kd = [kk * d for kk, d in zip(ks[j], D(j, last))]
        S = madd(S, outer(U[j], kd))
    return S


def deferred_run(variant, S0, qs, ks, vs, alphas, betas, L):
    """Base + bounded log of ``L`` slots, merged when full.

    Each step appends ``(k, v, alpha, beta)`` and reads out through the
    q-chain with every logged entry (the current one included); when the log
    holds ``L`` entries after the readout, it is merged into the base and
    emptied.  Returns ``(outputs, materialised final state, final fill)``.
    """
    base = [list(r) for r in S0]
    log = []
    outs = []
    for t in range(len(ks)):
        b = None if betas is None else betas[t]
        log.append((ks[t], vs[t], alphas[t], b))
        outs.append(qchain_readout(variant, base, log, qs[t]))
        if len(log) == L:
            base = wy_merge(variant, base, log)
            log = []
    fill = len(log)
    return outs, wy_merge(variant, base, log), fill


# ----------------------------------------------------------------------------
# additive-factor log
# ----------------------------------------------------------------------------
def af_append(variant, base, log, k, v, alpha, beta):
    """The next entry ``(a, b, P)`` of an additive-factor log.

    The log stands for the state ``base diag(P_c) + sum_j a_j (b_j * P_c / P_j)^T``
    (``P_j`` the decay accumulated over entries ``0..j``, ``c`` the newest):
    the dense base plus decayed rank-one terms, i.e. the compact update
    factors ``(a_t, b_t)`` with their log-decay snapshot of the DeltaLog
    page's Core Mechanism.  For a step with ``(k, v, alpha, beta)``:
    ``P_n = P_{n-1} * alpha``, ``b = k`` and ``a = beta (v - x)`` with
    ``x = S_{n-1} (alpha * k) = base (P_n * k) + sum_{j<n} a_j (b_j * P_n / P_j) . k``,
    read from base and log without materialising ``S_{n-1}`` (RWKV6: ``a = v``;
    gated: ``a = w * v - x`` with ``e * k`` in place of ``k`` in ``x``).
    """
    dk = len(k)
    prev = log[-1][2] if log else [Fr(1)] * dk
    Pn = [x * y for x, y in zip(prev, _chan(variant, alpha, dk))]
    kf = [Fr(x) for x in k]
    vf = [Fr(x) for x in v]
    if variant == RWKV6:
        return (vf, kf, Pn)
    rd = [Fr(e) * kk for e, kk in zip(beta[0], kf)] if variant == GDN2 else kf
    x = matvec(base, [p * kk for p, kk in zip(Pn, rd)])
    for a, b, Pj in log:
        u = sum((bb * p / pj * kk for bb, p, pj, kk in zip(b, Pn, Pj, rd)), Fr(0))
        x = [xi + u * ai for xi, ai in zip(x, a)]
    if variant == GDN2:
        return ([Fr(w) * vi - xi for w, vi, xi in zip(beta[1], vf, x)], kf, Pn)
    return ([Fr(beta) * (vi - xi) for vi, xi in zip(vf, x)], kf, Pn)


def af_readout(base, log, q):
    """``o = base (P_c * q) + sum_j a_j ((b_j * P_c / P_j) . q)``: independent
    dot products per entry, no triangular solve and no chain."""
    qf = [Fr(x) for x in q]
    if not log:
        return matvec(base, qf)
    Pc = log[-1][2]
    o = matvec(base, [p * x for p, x in zip(Pc, qf)])
    for a, b, Pj in log:
        r = sum((bb * p / pj * x for bb, p, pj, x in zip(b, Pc, Pj, qf)), Fr(0))
        o = [oi + r * ai for oi, ai in zip(o, a)]
    return o


def af_merge(base, log):
    """``base diag(P_c) + sum_j a_j (b_j * P_c / P_j)^T``: one contraction."""
    if not log:
        return [list(r) for r in base]
    Pc = log[-1][2]
    S = [[x * p for x, p in zip(row, Pc)] for row in base]
    for a, b, Pj in log:
        S = madd(S, outer(a, [bb * p / pj for bb, p, pj in zip(b, Pc, Pj)]))
    return S


def af_deferred_run(variant, S0, qs, ks, vs, alphas, betas, L):
    """:func:`deferred_run` with the additive-factor log: every step appends
    ``(a, b, P)`` and reads out with every entry (the new one included);
    a full log is merged and emptied.  Returns ``(outputs, final state, fill,
    every appended factor a in order)``."""
    base = [list(r) for r in S0]
    log, outs, factors = [], [], []
    for t in range(len(ks)):
        b = None if betas is None else betas[t]
        log.append(af_append(variant, base, log, ks[t], vs[t], alphas[t], b))
        factors.append(log[-1][0])
        outs.append(af_readout(base, log, qs[t]))
        if len(log) == L:
            base = af_merge(base, log)
            log = []
    return outs, af_merge(base, log), len(log), factors


def compact_wy_T(betas, ks):
    """``T`` with ``prod_j (I - beta_j k_j k_j^T) = I - K T K^T`` (K = [k_1..k_n]).

    Forward accumulation: ``T_jj = beta_j``,
    ``T[:j, j] = -beta_j T[:j, :j] K[:, :j]^T k_j``.
    """
    n = len(ks)
    T = [[Fr(0)] * n for _ in range(n)]
    for j in range(n):
        T[j][j] = Fr(betas[j])
        z = [dot(ks[i], ks[j]) for i in range(j)]
        for i in range(j):
            T[i][j] = -Fr(betas[j]) * sum((T[i][m] * z[m] for m in range(j)), Fr(0))
    return T


# ----------------------------------------------------------------------------
# schedule
# ----------------------------------------------------------------------------
def schedule(L, offset, steps):
    """Slot written and merge decision per step for one sequence.

    A sequence whose log already holds ``offset`` entries writes slot
    ``(offset + t) mod L`` at step ``t`` and is merged after that step iff
    ``(offset + t + 1) mod L == 0``.  Returns a list of
    ``(slot, merge_after, fill_after_step_and_merge)``.
    """
    out = []
    fill = offset
    for t in range(steps):
        slot = fill
        fill += 1
        merged = fill == L
        if merged:
            fill = 0
        out.append((slot, merged, fill))
    return out
