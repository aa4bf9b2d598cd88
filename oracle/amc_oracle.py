"""Float64 CPU oracle for attention-matching KV compaction (AM-OMP).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline of the benchmark may import this module.  It shares no code with the
HIP library: it is a plain, slow, obviously-correct restatement of what the
method computes, in float64, using numpy and scipy.

Citations name the web page and its section ("Fast KV Compaction via
Attention Matching", arXiv 2602.16284, as summarised on the pages):

* p1 = zhichai.net deep-dive (Chinese), sections 1.3 (mass), 1.4 (scalar
  bias), 1.6 (OMP key selection);
* p2 = xinfinite.net article, sections 1 (mixing identity and matching
  conditions) and 2 (three-step pipeline: step 2 key selection + NNLS bias
  fit, Fig. 2 projected-gradient NNLS; step 3 OLS value fit) and 3 (top-k
  batched selection with delayed refit, Table 1);
* p3 = zhichai.net English summary, "Key Points" and "The Three-Step
  Closed-Form Pipeline";
* p4 = youleyou.com news rewrite, "the math" section (output and mass
  matching, NNLS then OLS).

Readings where the pages are silent or garbled (each is also listed in the
design notes):

* logits carry the model's scale 1/sqrt(d) (the pages write exp(q.k));
* one per-head shift s = max logit is subtracted before exp; the selection,
  the NNLS minimiser and beta are invariant to it;
* beta = beta_in + log w (a key with w = 0 gets beta = -inf and value 0);
* the selection score is the signed, unnormalised r^T Phi[:, j]; ties go to
  the lower original index;
* between refits of the batched variant the new keys carry w = 0 and the
  residual is left as it was; a refit always follows the last key;
* the value fit is an unweighted, unregularised minimum-norm least squares on
  the keys with w > 0;
* output keys are sorted by original index.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
from scipy.optimize import nnls as _scipy_nnls

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# attention, mass, features
# ----------------------------------------------------------------------------
def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def logits(Q, K, bias=None, scale=None):
    """l_ij = scale * q_i . k_j + bias_j   (bias: per-key additive logit bias)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if scale is None:
        scale = default_scale(Q.shape[1])
    L = scale * (Q @ K.T)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def attention(Q, K, V, bias=None, scale=None):
    """Softmax attention output O and log attention mass log Mass(q).

    Mass(q; K) = sum_j exp(l_j) is the block's unnormalised attention weight
    (p1 section 1.3; p3 Key Points).  Returns (O [n, d_v], logM [n]).
    """
    L = logits(Q, K, bias, scale)
    mx = np.max(L, axis=1, keepdims=True)
    E = np.exp(L - mx)
    Z = E.sum(axis=1)
    O = (E @ np.asarray(V, dtype=np.float64)) / Z[:, None]
    return O, np.log(Z) + mx[:, 0]


def mix_blocks(O1, logM1, O2, logM2):
    """Output of attention over two concatenated blocks from the blocks' local
    outputs and masses: the mass-weighted mixture (p1 section 1.3; p2 section 1,
    the mixing identity)."""
    mx = np.maximum(logM1, logM2)
    a1 = np.exp(logM1 - mx)
    a2 = np.exp(logM2 - mx)
    return (a1[:, None] * O1 + a2[:, None] * O2) / (a1 + a2)[:, None], mx + np.log(a1 + a2)


@dataclass
class Features:
    Phi: np.ndarray  # (n, T) exp(l - s)
    m: np.ndarray  # (n,)  Phi @ 1
    Y: np.ndarray  # (n, d_v) (Phi @ V) / m
    shift: float


def mass_features(Q, K, V, bias=None, scale=None, shift=None) -> Features:
    """Mass feature matrix Phi_ij = exp(l_ij - s), target mass m = Phi 1
    (p1 section 1.6) and the original attention output Y = Phi V / m, the
    value-fit target (p2 section 2, step 3)."""
    L = logits(Q, K, bias, scale)
    s = float(np.max(L)) if shift is None else float(shift)
    Phi = np.exp(L - s)
    m = Phi.sum(axis=1)
    Y = (Phi @ np.asarray(V, dtype=np.float64)) / m[:, None]
    return Features(Phi, m, Y, s)


# ----------------------------------------------------------------------------
# NNLS
# ----------------------------------------------------------------------------
def nnls_lawson_hanson(A, y):
    """min_{w >= 0} ||A w - y||_2 by Lawson and Hanson's active-set method
    (scipy's implementation)."""
    w, _ = _scipy_nnls(np.asarray(A, dtype=np.float64), np.asarray(y, dtype=np.float64), maxiter=50 * A.shape[1] + 50)
    return w


def fnnls(G, b, w0=None, tol=None, max_outer=None):
    """min_{w >= 0} 0.5 w^T G w - b^T w for symmetric positive definite G, by
    Bro and De Jong's fast active-set NNLS ("FNNLS", J. Chemometrics 1997),
    which works on the Gram form G = A^T A, b = A^T y.

    The problem is first put in unit-diagonal form (w = D u with
    D = diag(G)^-1/2, which maps u >= 0 onto w >= 0, so the minimiser is the
    same); the tolerance on the gradient is then meaningful for every column
    however different the column norms are.

    ``w0`` is an optional feasible warm start (w0 >= 0); the passive set starts
    as its support.  The minimiser is unique for G positive definite, so the
    warm start does not change the answer.
    """
    G = np.asarray(G, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    t = b.shape[0]
    dg = np.sqrt(np.diag(G))
    dg = np.where(dg > 0, dg, 1.0)
    Gs = G / dg[:, None] / dg[None, :]
    bs = b / dg
    if tol is None:
        tol = 10.0 * np.finfo(np.float64).eps * max(1e-300, np.max(np.abs(bs))) * t
    if max_outer is None:
        max_outer = 30 * t + 30
    u = np.zeros(t) if w0 is None else np.maximum(np.asarray(w0, dtype=np.float64), 0.0) * dg
    passive = u > 0

    def solve_passive(u, passive):
        # least squares on the passive set; step back toward u while any
        # passive variable would turn non-positive, dropping the blocking one
        while np.any(passive):
            P = np.flatnonzero(passive)
            z = np.zeros(t)
            z[P] = np.linalg.solve(Gs[np.ix_(P, P)], bs[P])
            if np.all(z[P] > 0):
                return z, passive
            neg = P[z[P] <= 0]
            ratios = u[neg] / (u[neg] - z[neg])
            i_min = int(np.argmin(ratios))
            u = u + ratios[i_min] * (z - u)
            u[neg[i_min]] = 0.0
            passive = passive & (u > 0)
            u[~passive] = 0.0
        return np.zeros(t), passive

    if np.any(passive):
        u, passive = solve_passive(u, passive)
    for _ in range(max_outer):
        g = bs - Gs @ u  # negative gradient
        cand = np.where(~passive, g, -np.inf)
        j = int(np.argmax(cand))
        if cand[j] <= tol:
            return u / dg
        passive = passive.copy()
        passive[j] = True
        u, passive = solve_passive(u, passive)
    raise RuntimeError(f"fnnls: no KKT point within {max_outer} outer iterations")


def _householder_r(M):
    """Upper-triangular factor R of M = QR by Householder reflections, for
    dtypes numpy's LAPACK binding does not take (extended precision)."""
    A = np.array(M, copy=True)
    rows, cols = A.shape
    for j in range(min(rows, cols)):
        x = A[j:, j]
        nrm = np.sqrt(np.sum(x * x))
        if nrm == 0:
            continue
        alpha = -nrm if x[0] >= 0 else nrm
        v = x.copy()
        v[0] -= alpha
        vtv = np.sum(v * v)
        A[j:, j:] -= np.outer(v, (v @ A[j:, j:]) * (2 / vtv))
        A[j + 1:, j] = 0
    return A[:min(rows, cols)]


def _qr_r(M):
    M = np.asarray(M)
    if M.dtype == np.float64:
        return np.linalg.qr(M, mode="r")
    return _householder_r(M)


# Lawson-Hanson on the reduced system: a zero column enters when its part
# orthogonal to the free columns makes a cosine above COS_TOL with the
# residual; a column whose orthogonal part is below DEP_TOL (unit columns)
# counts as dependent on the free set.
COS_TOL = 1e-10
DEP_TOL = 1e-12
KKT_ACCEPT = 1e-8  # largest relative KKT violation of scipy's Lawson-Hanson result kept by nnls_exact
STALL_ENTERS = 64  # nnls_lh_update: entering steps over which ...
STALL_REL = 1e-15  # ... the residual must fall by more than this fraction of |m| to go on


def nnls_qr(PhiS, m, w0=None, max_outer=None, dtype=np.float64):
    """min_{w >= 0} ||Phi_S w - m||_2 by Lawson and Hanson's active-set method,
    with every least-squares step taken through an orthogonal factorisation
    of Phi_S itself, never its Gram matrix (whose conditioning is the square
    of Phi_S's, the whole difference when the selected keys are nearly
    collinear and the mass is almost fitted).

    1. Columns are scaled to unit norm (w = u / ||phi_j||, a bijection of the
       non-negative orthant, so the minimiser is the same) and [Phi_S D^-1 m]
       is reduced to its triangular factor [[A y] [0 rho]]: for every u,
       ||Phi_S D^-1 u - m||^2 = ||A u - y||^2 + rho^2, so the problem is
       min_{u >= 0} ||A u - y|| with A square upper triangular.
    2. Each active-set iteration factors the columns of A ordered [free | zero]
       next to y.  The leading block gives the least-squares solution on the
       free set; the trailing block holds the residual and every zero
       column's component orthogonal to the free columns.  A free variable
       that would turn non-positive makes the usual Lawson-Hanson step back
       to feasibility and leaves; otherwise the zero column whose orthogonal
       component is best aligned with the residual enters (the entering test
       of Lawson and Hanson, measured in the complement, where rounding is
       relative to the residual rather than to m).

    ``w0``: optional feasible warm start; its support is the starting free
    set.  The minimiser is unique when Phi_S has full column rank, so the
    warm start does not change it.  ``dtype``: arithmetic of the solve
    (numpy.longdouble for an extended-precision cross-check).
    """
    A0 = np.asarray(PhiS, dtype=dtype)
    y0 = np.asarray(m, dtype=dtype)
    n, t = A0.shape
    dg = np.sqrt(np.sum(A0 * A0, axis=0))
    live = dg > 0
    dg = np.where(live, dg, 1)
    R = _qr_r(np.column_stack([A0 / dg, y0]))
    A = np.zeros((t, t), dtype=dtype)
    y = np.zeros(t, dtype=dtype)
    k = min(R.shape[0], t)
    A[:k] = R[:k, :t]
    y[:k] = R[:k, t]
    if max_outer is None:
        max_outer = 3 * t + 30
    u = np.zeros(t, dtype=dtype)
    if w0 is not None:
        u[: len(w0)] = np.maximum(np.asarray(w0, dtype=dtype), 0) * dg[: len(w0)]
    u[~live] = 0
    free = [a for a in range(t) if u[a] > 0]
    blocked = set(np.flatnonzero(~live).tolist())
    for _ in range(max_outer):
        zero = [a for a in range(t) if u[a] == 0 and a not in blocked and a not in free]
        f = len(free)
        T = _qr_r(np.column_stack([A[:, free + zero], y]))
        Tf = np.zeros((t, t + 1), dtype=dtype)
        Tf[: T.shape[0], : T.shape[1]] = T  # fewer columns once some are left out
        c = Tf[:, f + len(zero)]
        dep = [i for i in range(f) if abs(Tf[i, i]) <= DEP_TOL]
        if dep:  # dependent on the free columns before it: out for good
            a = free[dep[0]]
            blocked.add(a)
            u[a] = 0
            free.remove(a)
            continue
        z = np.zeros(f, dtype=dtype)
        for i in range(f - 1, -1, -1):
            z[i] = (c[i] - Tf[i, i + 1:f] @ z[i + 1:]) / Tf[i, i]
        if np.any(z <= 0):
            # step from the feasible u toward z until the first free variable hits zero
            neg = np.flatnonzero(z <= 0)
            uf = u[free]
            ratios = uf[neg] / (uf[neg] - z[neg])
            i_min = int(neg[int(np.argmin(ratios))])
            uf = uf + ratios.min() * (z - uf)
            uf[i_min] = 0
            u[free] = np.maximum(uf, 0)
            free = [a for a in free if u[a] > 0]
            continue
        u[:] = 0
        u[free] = z
        rz = c[f:]
        nr = np.sqrt(np.sum(rz * rz))
        best, enter = COS_TOL, -1
        for q, a in enumerate(zero):
            col = Tf[f:f + q + 1, f + q]
            den = np.sqrt(np.sum(col * col))
            if den <= DEP_TOL or nr == 0:
                continue
            cos = (col @ rz[: q + 1]) / (den * nr)
            if cos > best:
                best, enter = cos, a
        if enter < 0:
            return (u / dg).astype(np.float64)
        free.append(enter)
    raise RuntimeError(f"nnls_qr: no KKT point within {max_outer} iterations")


def nnls_lh_update(PhiS, m, w0=None, max_outer=None, dtype=np.float64):
    """nnls_qr's Lawson-Hanson iteration, step for step, with the factor of
    the columns ordered [free | zero] and y kept from one iteration to the
    next instead of recomputed (the same algorithm: p1 section 1.6, the NNLS
    refit; its least-squares steps through an orthogonal factorisation of
    Phi_S).  O(t^2) per iteration instead of nnls_qr's O(t^3), for budgets in
    the thousands.

    State: W (t rows; columns in position order, the free block upper
    triangular, zero columns full height) and c, both Q^T of the reduced
    system for some orthogonal Q.
    - A column enters: it moves to position f and one Householder reflection
      of rows f..t-1 zeroes it below row f (the zero columns and c take it).
    - A column leaves from free position k: the free columns after it move
      down one place and a Givens rotation of rows q, q+1 for q = k..f-2
      restores the triangle (every column from q on and c take them); a
      column kept for later goes to the zero block, a dependent one is
      dropped.
    Norms of the zero columns below row f and their inner products with c
    there do not depend on Q, so the entering test is nnls_qr's; ties go to
    the lower key, as there.  Near a degenerate minimiser float64 can keep
    swapping columns at the rounding level (each entering column's cosine
    near 1e-6, the residual moving in its twelfth digit, far below the
    resolution eps |m| of a float64 residual) until the iteration cap: there,
    when the last STALL_ENTERS entering steps lowered the residual by less
    than STALL_REL |m|, the iterate is the minimiser to float64 resolution
    and is returned (otherwise the cap is an error).  Every other run ends
    where nnls_qr's does.
    ``dtype``: arithmetic of the solve (numpy.longdouble for an
    extended-precision cross-check; STALL_REL then scales with its epsilon).
    """
    from scipy.linalg import solve_triangular

    A0 = np.asarray(PhiS, dtype=dtype)
    y0 = np.asarray(m, dtype=dtype)
    wide = np.dtype(dtype) != np.float64
    stall = STALL_REL * float(np.finfo(dtype).eps / np.finfo(np.float64).eps)

    def back_sub(Tm, b):
        if not wide:
            return solve_triangular(Tm, b, check_finite=False)
        z = np.zeros(len(b), dtype=dtype)
        for i in range(len(b) - 1, -1, -1):
            z[i] = (b[i] - Tm[i, i + 1:] @ z[i + 1:]) / Tm[i, i]
        return z

    n, t = A0.shape
    dg = np.sqrt(np.sum(A0 * A0, axis=0))
    live = dg > 0
    dg = np.where(live, dg, 1)
    R = _qr_r(np.column_stack([A0 / dg, y0]))
    A = np.zeros((t, t), dtype=dtype)
    y = np.zeros(t, dtype=dtype)
    k0 = min(R.shape[0], t)
    A[:k0] = R[:k0, :t]
    y[:k0] = R[:k0, t]
    if max_outer is None:
        max_outer = 3 * t + 30
    u = np.zeros(t, dtype=dtype)
    if w0 is not None:
        u[: len(w0)] = np.maximum(np.asarray(w0, dtype=dtype), 0) * dg[: len(w0)]
    u[~live] = 0
    free = [a for a in range(t) if u[a] > 0]
    zero = [a for a in range(t) if live[a] and u[a] == 0]
    Mf = _qr_r(np.column_stack([A[:, free + zero], y]))
    ncol = len(free) + len(zero)  # live columns of W (positions 0..ncol-1)
    W = np.zeros((t, max(ncol, 1)), dtype=dtype)
    c = np.zeros(t, dtype=dtype)
    W[: Mf.shape[0], :ncol] = Mf[:, :-1]
    c[: Mf.shape[0]] = Mf[:, -1]
    cols = free + zero  # key of each column position
    hist = []  # residual norm at each feasible solve
    ym = np.sqrt(np.sum(y0 * y0))

    def leave(k, keep):
        # the free columns after k move down one place (the leaving column
        # to position f - 1, the first zero place, or out when not kept)
        nonlocal ncol
        f = len(free)
        key = cols[k]
        colk = W[:, k].copy()
        W[:, k: f - 1] = W[:, k + 1: f]
        W[:, f - 1] = colk
        del cols[k]
        cols.insert(f - 1, key)
        del free[k]
        if keep:
            zero.append(key)
        else:  # dropped: to the last live place, then out
            W[:, [f - 1, ncol - 1]] = W[:, [ncol - 1, f - 1]]
            cols[f - 1], cols[ncol - 1] = cols[ncol - 1], cols[f - 1]
            cols.pop()
            ncol -= 1
        for q in range(k, f - 1):
            a, b = W[q, q], W[q + 1, q]
            r = np.hypot(a, b)
            if r == 0.0:
                continue
            cs, sn = a / r, b / r
            top = W[q, q:ncol].copy()
            W[q, q:ncol] = cs * top + sn * W[q + 1, q:ncol]
            W[q + 1, q:ncol] = cs * W[q + 1, q:ncol] - sn * top
            W[q + 1, q] = 0.0
            cq = c[q]
            c[q] = cs * cq + sn * c[q + 1]
            c[q + 1] = cs * c[q + 1] - sn * cq

    for _ in range(max_outer):
        f = len(free)
        d = np.abs(np.diag(W[:f, :f])) if f else np.zeros(0)
        dep = np.flatnonzero(d <= DEP_TOL)
        if dep.size:  # dependent on the free columns before it: out for good
            a = free[int(dep[0])]
            u[a] = 0
            leave(int(dep[0]), False)
            continue
        z = back_sub(W[:f, :f], c[:f]) if f else np.zeros(0, dtype=dtype)
        if np.any(z <= 0):
            # step from the feasible u toward z until the first free variable hits zero
            neg = np.flatnonzero(z <= 0)
            uf = u[free]
            ratios = uf[neg] / (uf[neg] - z[neg])
            i_min = int(neg[int(np.argmin(ratios))])
            uf = uf + ratios.min() * (z - uf)
            uf[i_min] = 0
            u[free] = np.maximum(uf, 0)
            for kk in range(f - 1, -1, -1):
                if not u[free[kk]] > 0:
                    leave(kk, True)
            continue
        u[:] = 0
        u[free] = z
        rz = c[f:]
        nr = np.sqrt(np.sum(rz * rz))
        nz = ncol - f
        hist.append(nr)
        enter = -1
        if nz and nr > 0:
            Z = W[f:, f:ncol]
            den = np.sqrt(np.einsum("ij,ij->j", Z, Z))
            with np.errstate(invalid="ignore", divide="ignore"):
                cos = np.where(den > DEP_TOL, (rz @ Z) / (den * nr), -np.inf)
            best = np.max(cos)
            if best > COS_TOL:
                keys = np.asarray(cols[f:ncol])
                enter = f + int(np.flatnonzero(cos == best)[np.argmin(keys[cos == best])])
        if enter < 0:
            return (u / dg).astype(np.float64)
        # the entering column to position f, then one reflection of rows f..t-1
        key = cols[enter]
        W[:, [f, enter]] = W[:, [enter, f]]
        cols[f], cols[enter] = cols[enter], cols[f]
        zero.remove(key)
        free.append(key)
        x = W[f:, f]
        nrm = np.sqrt(np.sum(x * x))
        if nrm > 0 and f + 1 < t:
            alpha = -nrm if x[0] >= 0 else nrm
            v = x.copy()
            v[0] -= alpha
            vtv = np.sum(v * v)
            if vtv > 0:
                B = W[f:, f:ncol]
                B -= np.multiply.outer(v, (v @ B) * (2 / vtv))
                c[f:] -= v * ((v @ c[f:]) * (2 / vtv))
                W[f + 1:, f] = 0.0
    if len(hist) > STALL_ENTERS and hist[-1 - STALL_ENTERS] - hist[-1] <= stall * ym:
        return (u / dg).astype(np.float64)  # swapping at the rounding level (see above)
    raise RuntimeError(f"nnls_lh_update: no KKT point within {max_outer} iterations")


def nnls_exact(PhiS, m, w_prev=None):
    """The exact NNLS minimiser of ||Phi_S w - m|| over w >= 0, the bias fit of
    the key-selection step (p1 section 1.6: refit w by NNLS; p2 section 2,
    step 2; p4: with C_k fixed the mass matching is an NNLS problem).

    The pages' GPU solver is projected gradient (p2 Fig. 2); what it converges
    to is this minimiser, which the oracle computes directly: Lawson-Hanson
    (scipy) for up to 256 columns, above that Lawson-Hanson on the
    triangular factor of [Phi_S m] with the factor updated between
    iterations (nnls_lh_update, nnls_qr's iteration), warm-started from the
    previous refit's weights.  Both work on Phi_S through orthogonal
    factorisations.
    """
    t = PhiS.shape[1]
    if t <= 256:
        # scipy's result is kept only where it meets the optimality conditions:
        # on a rank-deficient system (fewer queries than keys) it can stop
        # short of the minimiser, and nnls_qr then solves it
        w = nnls_lawson_hanson(PhiS, m)
        A = np.asarray(PhiS, dtype=np.float64)
        if nnls_kkt_violation(A.T @ A, A.T @ np.asarray(m, dtype=np.float64), w) <= KKT_ACCEPT:
            return w
        return nnls_qr(PhiS, m)
    w0 = None
    if w_prev is not None:
        w0 = np.zeros(t)
        w0[: len(w_prev)] = w_prev
    return nnls_lh_update(PhiS, m, w0)


def nnls_kkt_violation(G, b, w):
    """Largest violation of the NNLS optimality conditions in unit-diagonal
    form (column j scaled by 1/sqrt(G_jj)), relative to the largest scaled
    |b_j|: w >= 0, the gradient g = G w - b vanishes where w > 0 and is
    non-negative where w = 0."""
    G = np.asarray(G, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dg = np.sqrt(np.diag(G))
    dg = np.where(dg > 0, dg, 1.0)
    g = (G @ w - b) / dg
    scale = max(np.max(np.abs(b / dg)), 1e-300)
    v_neg = max(0.0, -np.min(w * dg)) / scale if w.size else 0.0
    act = w > 0
    v_free = np.max(np.abs(g[act])) if np.any(act) else 0.0
    v_bound = max(0.0, -np.min(g[~act])) if np.any(~act) else 0.0
    return max(v_neg, v_free / scale, v_bound / scale)


# ----------------------------------------------------------------------------
# OMP key selection (with the batched / lazy-refit variant)
# ----------------------------------------------------------------------------
@dataclass
class Step:
    it: int  # 1-based iteration number
    picks: List[int]  # original key indices chosen at this iteration
    scores: List[float]  # oracle scores of the picks
    runner_up: float  # best score not picked
    top: float  # best score at this iteration
    margin: float  # (score of last pick - runner_up) / |top|
    refit: bool
    forced: bool = False  # replay: the oracle followed the caller's picks in a tie zone
    mismatch: bool = False  # replay: caller's picks differ where the margin is clear
    resid_norm: float = float("nan")


@dataclass
class Selection:
    S: List[int]  # selection order
    w: np.ndarray  # weights in selection order
    r: np.ndarray  # final residual m - Phi_S w
    steps: List[Step] = field(default_factory=list)


def iteration_sizes(t: int, k: int, R: int):
    """Number of keys taken at each iteration and whether a refit follows it:
    kk = min(k, t - |S|); refit when it mod R == 0 or |S| == t."""
    out = []
    size, it = 0, 0
    while size < t:
        it += 1
        kk = min(k, t - size)
        size += kk
        out.append((kk, (it % R == 0) or size == t))
    return out


def _rank(c):
    """Indices ordered by score descending, ties to the lower index."""
    return np.lexsort((np.arange(c.shape[0]), -c))


def omp_select(Phi, m, t, k=1, R=1, replay: Optional[Sequence[Sequence[int]]] = None,
               margin_tol: float = 1e-6, tie_ulps: float = 0.0) -> Selection:
    """Greedy OMP key selection with NNLS refits (p1 section 1.6).

    r = m, S = {}.  Each iteration scores every unselected key by r^T Phi[:, j]
    and takes the best (the plain method, k = R = 1) or the best kk = min(k,
    t - |S|) (top-k batched selection, p2 section 3; p3 "AM-OMP-Batch").  After
    the iteration the weights are refit by exact NNLS and r = m - Phi_S w,
    every R-th iteration and after the last one (delayed refit, p2 section 3).

    ``replay``: per-iteration picks of another implementation.  Where the
    oracle's own margin exceeds ``margin_tol`` the picks must equal the
    oracle's (a mismatch is recorded); the oracle then follows the given
    picks either way, so later steps share the same history.

    ``tie_ulps``: the float64 resolution of the scores.  r = m - Phi_S w is a
    difference of nearly equal sums, so each score c_j carries a rounding
    error up to about tie_ulps * eps * (Phi[:, j]^T m) (summation bounds for
    r and c, plus the ulp-level differences two implementations' exp and
    logits leave in Phi).  A replayed pick whose oracle score lies within the
    two keys' bounds of the oracle's own pick is a tie, whatever the relative
    margin: once the mass is fitted to ~1e-9 these bounds exceed 1e-6 of the
    top score, and no float64 computation decides those picks.
    """
    Phi = np.asarray(Phi, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    n, T = Phi.shape
    if not (1 <= t <= T):
        raise ValueError("budget must satisfy 1 <= t <= T")
    S: List[int] = []
    w = np.zeros(0)
    r = m.copy()
    steps: List[Step] = []
    selected = np.zeros(T, dtype=bool)
    b_all = np.abs(Phi).T @ np.abs(m)  # scale of each score's rounding error
    for it, (kk, refit) in enumerate(iteration_sizes(t, k, R), start=1):
        c = Phi.T @ r
        c[selected] = NEG_INF
        order = _rank(c)
        picks = [int(j) for j in order[:kk]]
        remaining = T - len(S)
        runner = float(c[order[kk]]) if kk < remaining else NEG_INF
        top = float(c[order[0]])
        last = float(c[order[kk - 1]])
        if runner == NEG_INF:
            margin = np.inf
        elif top == 0.0:
            margin = 0.0 if last == runner else np.inf
        else:
            margin = (last - runner) / abs(top)
        st = Step(it, picks, [float(c[j]) for j in picks], runner, top, margin, refit)
        if replay is not None:
            given = [int(j) for j in replay[it - 1]]
            if len(given) != kk or len(set(given)) != kk or any(selected[j] for j in given):
                raise ValueError(f"replay iteration {it}: invalid picks {given}")
            if set(given) != set(picks):
                # the given set differs from the oracle's: it is a different
                # selection if some key left out scores above some given key
                # by more than both the margin and the two keys' rounding
                # bounds (then no ordering within float64 resolution makes
                # the given set a top kk)
                eb = tie_ulps * np.finfo(np.float64).eps
                out = ~selected
                out[given] = False
                c_out, b_out = c[out], b_all[out]
                thr = margin_tol * abs(top)
                resolved = any(np.any((c_out - c[g] > thr) & (c_out - c[g] > eb * (b_out + b_all[g]))) for g in given)
                if resolved:
                    st.mismatch = True
                else:
                    st.forced = True
            picks = given
            st.picks = given
            st.scores = [float(c[j]) for j in given]
        for j in picks:
            selected[j] = True
        S.extend(picks)
        w = np.concatenate([w, np.zeros(kk)])
        if refit:
            PhiS = Phi[:, S]
            w = nnls_exact(PhiS, m, w_prev=w)
            r = m - PhiS @ w
        st.resid_norm = float(np.linalg.norm(r))
        steps.append(st)
    return Selection(S, w, r, steps)


def highest_scores(Phi, m):
    """AM-Highest key scores (p3 "Method Family and Trade-offs": highest-
    attention key selection; p4, the highest-attention-keys method): each
    key's attention summed over the reference queries, sum_i Phi_ij / m_i
    (row i of Phi divided by its mass is query i's softmax over the keys)."""
    Phi = np.asarray(Phi, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    return (Phi / m[:, None]).sum(axis=0)


def highest_select(Phi, m, t, given=None, margin_tol: float = 1e-6) -> Selection:
    """AM-Highest: the t keys with the largest highest_scores (ties to the
    lower index), then one exact NNLS refit of their weights.

    ``given``: another implementation's key set.  Where a key it leaves out
    scores above a key it takes by more than ``margin_tol`` of the top score
    the step is a mismatch; the oracle then continues with the given set (so
    the weights and values that follow are compared on the same keys)."""
    c = highest_scores(Phi, m)
    T = c.shape[0]
    if not (1 <= t <= T):
        raise ValueError("budget must satisfy 1 <= t <= T")
    order = _rank(c)
    picks = [int(j) for j in order[:t]]
    top = float(c[order[0]])
    runner = float(c[order[t]]) if t < T else NEG_INF
    last = float(c[order[t - 1]])
    margin = np.inf if runner == NEG_INF else ((last - runner) / abs(top) if top != 0.0 else 0.0)
    st = Step(1, picks, [float(c[j]) for j in picks], runner, top, margin, True)
    if given is not None:
        g = [int(j) for j in given]
        if len(g) != t or len(set(g)) != t:
            raise ValueError("given: invalid key set")
        out = np.ones(T, dtype=bool)
        out[g] = False
        thr = margin_tol * abs(top)
        c_in_min = min(float(c[j]) for j in g)
        if np.any(c[out] - c_in_min > thr):
            st.mismatch = True
        elif set(g) != set(picks):
            st.forced = True
        picks = g
        st.picks = g
        st.scores = [float(c[j]) for j in g]
    S = picks
    w = nnls_exact(np.asarray(Phi, dtype=np.float64)[:, S], m)
    r = np.asarray(m, dtype=np.float64) - np.asarray(Phi, dtype=np.float64)[:, S] @ w
    return Selection(S, w, r, [st])


# ----------------------------------------------------------------------------
# OLS value fit
# ----------------------------------------------------------------------------
def ols_values(PhiS, w, Y):
    """Compacted values C_v (p2 section 2, step 3; p3 pipeline step 3; p4).

    With C_k and beta fixed, the compacted block's attention output for query
    i is sum_j A_ij C_v[j] with A_ij = Phi_S[i, j] w_j / mhat_i and
    mhat = Phi_S w; C_v minimises ||A C_v - Y||_F (ordinary least squares,
    minimum norm, on the keys with w > 0; keys with w = 0 get C_v = 0).
    """
    PhiS = np.asarray(PhiS, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    F = w > 0
    mhat = PhiS @ w
    A = PhiS[:, F] * w[F][None, :] / mhat[:, None]
    Cv = np.zeros((w.shape[0], Y.shape[1]))
    if np.any(F):
        Cv[F] = np.linalg.lstsq(A, Y, rcond=None)[0]
    return Cv


# ----------------------------------------------------------------------------
# the whole per-head compaction
# ----------------------------------------------------------------------------
@dataclass
class Compaction:
    sel_idx: np.ndarray  # (t,) ascending original indices
    Ck: np.ndarray  # (t, d) = K[sel_idx]
    beta: np.ndarray  # (t,)
    Cv: np.ndarray  # (t, d)
    w: np.ndarray  # (t,) NNLS weights, ascending-index order
    selection: Selection
    features: Features


def log_weights(w):
    with np.errstate(divide="ignore"):
        return np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), NEG_INF)


def score_tie_ulps(Q, K, t, beta_in=None, scale=None):
    """Rounding bound of the selection scores, in units of eps * (Phi[:, j]^T m):
    2 (t + 1) for the sums that form r and c, plus 2 (max |logit| + 2) for
    the ulp differences of Phi between two float64 implementations (a logit
    error of eps |l| becomes a relative error of Phi)."""
    L = logits(Q, K, beta_in, scale)
    return 2.0 * (t + 1) + 2.0 * (float(np.max(np.abs(L[np.isfinite(L)]))) + 2.0)


def compact(Q, K, V, t, k=1, R=1, beta_in=None, scale=None, shift=None, replay=None,
            margin_tol=1e-6, select: str = "omp") -> Compaction:
    """Compact one head's (K, V) to t keys: C_k (a subset of K), per-key bias
    beta and fitted values C_v (p2 section 2; p3 pipeline).  select: "omp"
    (greedy OMP, plain or batched by k and R) or "highest" (AM-Highest; k, R
    unused; ``replay`` is then the other implementation's key set)."""
    K = np.asarray(K, dtype=np.float64)
    feats = mass_features(Q, K, V, beta_in, scale, shift)
    if select == "highest":
        sel = highest_select(feats.Phi, feats.m, t, replay, margin_tol)
    else:
        tie = score_tie_ulps(Q, K, t, beta_in, scale) if replay is not None else 0.0
        sel = omp_select(feats.Phi, feats.m, t, k, R, replay, margin_tol, tie)
    S = np.asarray(sel.S, dtype=np.int64)
    Cv = ols_values(feats.Phi[:, S], sel.w, feats.Y)
    beta = log_weights(sel.w)
    if beta_in is not None:
        beta = beta + np.asarray(beta_in, dtype=np.float64)[S]
    order = np.argsort(S, kind="stable")
    return Compaction(S[order], K[S[order]], beta[order], Cv[order], sel.w[order], sel, feats)


def chunk_budgets(T: int, t: int, chunk_keys: int):
    """KV-based chunked compaction's split (p2 section 3, chunked compression:
    the prefilled KV is sliced into consecutive chunks, each compacted on its
    own; p1 section 4.3): chunks [c L, min((c+1) L, T)) of L = chunk_keys keys,
    and budget t shared in proportion to the chunks' lengths by largest
    remainders (ties to the earlier chunk), each at least 1 and at most its
    length.  Returns [(k0, k1, t_c)]."""
    if not (1 <= t <= T) or chunk_keys < 1:
        raise ValueError("need 1 <= t <= T and chunk_keys >= 1")
    bounds = [(k0, min(k0 + chunk_keys, T)) for k0 in range(0, T, chunk_keys)]
    if t < len(bounds):
        raise ValueError("budget below one key per chunk")
    quota = [t * (k1 - k0) / T for k0, k1 in bounds]
    base = [max(1, min(k1 - k0, int(np.floor(q)))) for (k0, k1), q in zip(bounds, quota)]
    left = t - sum(base)
    order = sorted(range(len(bounds)), key=lambda c: (-(quota[c] - np.floor(quota[c])), c))
    while left != 0:
        moved = False
        for c in order:
            k0, k1 = bounds[c]
            if left > 0 and base[c] < k1 - k0:
                base[c] += 1
                left -= 1
                moved = True
            elif left < 0 and base[c] > 1:
                base[c] -= 1
                left += 1
                moved = True
            if left == 0:
                break
        if not moved:
            raise ValueError("no feasible split")
    return [(k0, k1, tc) for (k0, k1), tc in zip(bounds, base)]


@dataclass
class ChunkedCompaction:
    sel_idx: np.ndarray  # (t,) ascending original indices
    Ck: np.ndarray
    beta: np.ndarray
    Cv: np.ndarray
    chunks: List[Compaction]  # per chunk, indices within the chunk
    split: List[tuple]  # (k0, k1, t_c)


def compact_chunked(Q, K, V, t, chunk_keys, k=1, R=1, beta_in=None, scale=None, select: str = "omp",
                    replay=None, margin_tol=1e-6) -> ChunkedCompaction:
    """KV-based chunked compaction: each chunk of chunk_keys consecutive keys
    compacted against the same reference queries (its own shift, features and
    fits), the compacted chunks concatenated in key order.  By the mixing
    identity (p1 section 1.3) attention over the concatenation combines the
    chunks' outputs by their masses, so each chunk matching its own output and
    mass makes the concatenation match the whole block's.  ``replay``: per
    chunk, what ``compact`` takes."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    split = chunk_budgets(K.shape[0], t, chunk_keys)
    parts = []
    for c, (k0, k1, tc) in enumerate(split):
        bi = None if beta_in is None else np.asarray(beta_in, dtype=np.float64)[k0:k1]
        parts.append(compact(Q, K[k0:k1], V[k0:k1], tc, k, R, beta_in=bi, scale=scale, select=select,
                             replay=None if replay is None else replay[c], margin_tol=margin_tol))
    sel = np.concatenate([p.sel_idx + k0 for p, (k0, _, _) in zip(parts, split)])
    return ChunkedCompaction(sel, np.concatenate([p.Ck for p in parts]), np.concatenate([p.beta for p in parts]),
                             np.concatenate([p.Cv for p in parts]), parts, split)


def greedy_swap_budgets(loss, unit: int, total: int):
    """Non-uniform head budgets by greedy swaps (p1 section 4.2; p2 section 4,
    Fig. 3 and 4): loss[h][j] is head h's sensitivity when it keeps (j+1)
    units of ``unit`` keys.  Every head starts even (the remainder one unit to
    each of the lowest heads); then, while a move lowers the summed loss, one
    unit goes to the head whose loss falls most by gaining it, from the other
    head whose loss rises least by losing it (ties to the lower head).
    Returns (budgets in keys, moves)."""
    L = np.asarray(loss, dtype=np.float64)
    H, J = L.shape
    if total % unit:
        raise ValueError("total must be a multiple of unit")
    units = total // unit
    if not (H <= units <= H * J):
        raise ValueError("total out of range")
    u = [units // H + (1 if h < units % H else 0) for h in range(H)]
    moves = 0
    while True:
        gains = [(L[h, u[h] - 1] - L[h, u[h]], h) for h in range(H) if u[h] < J]
        if not gains:
            break
        gain, r = max(gains, key=lambda x: (x[0], -x[1]))
        costs = [(L[h, u[h] - 2] - L[h, u[h] - 1], h) for h in range(H) if h != r and u[h] > 1]
        if not costs:
            break
        cost, d = min(costs, key=lambda x: (x[0], x[1]))
        if not gain > cost:
            break
        u[d] -= 1
        u[r] += 1
        moves += 1
    return [x * unit for x in u], moves


# ----------------------------------------------------------------------------
# error metrics (shift invariant)
# ----------------------------------------------------------------------------
def errors(Q, K, V, Ck, beta, Cv, beta_in=None, scale=None):
    """Relative mass error ||Mhat - M|| / ||M|| and relative attention-output
    error ||Ohat - O||_F / ||O||_F of a compacted block on the queries Q."""
    O, logM = attention(Q, K, V, beta_in, scale)
    Oc, logMc = attention(Q, Ck, Cv, beta, scale)
    s = np.max(logM)
    M = np.exp(logM - s)
    Mc = np.exp(logMc - s)
    e_mass = float(np.linalg.norm(Mc - M) / np.linalg.norm(M))
    e_out = float(np.linalg.norm(Oc - O) / np.linalg.norm(O))
    return e_mass, e_out


# ----------------------------------------------------------------------------
# online compaction schedule (p1 section 2.4; p2 section 5, Table 3)
# ----------------------------------------------------------------------------
def online_effective_length(physical: int, keep_newest: int, rounds: int, ratio: float = 0.5) -> int:
    """Tokens represented by a fixed physical cache after ``rounds`` online
    compactions: whenever the cache is full, everything but the newest
    ``keep_newest`` tokens is compacted by ``ratio`` and decoding refills it."""
    represented = physical
    for _ in range(rounds):
        old = physical - keep_newest
        freed = old - int(round(old * ratio))
        represented += freed
    return represented
