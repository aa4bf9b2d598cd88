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
            break
        passive = passive.copy()
        passive[j] = True
        u, passive = solve_passive(u, passive)
    return u / dg


def nnls_exact(PhiS, m, w_prev=None):
    """The exact NNLS minimiser of ||Phi_S w - m|| over w >= 0, the bias fit of
    the key-selection step (p1 section 1.6: refit w by NNLS; p2 section 2,
    step 2; p4: with C_k fixed the mass matching is an NNLS problem).

    The pages' GPU solver is projected gradient (p2 Fig. 2); what it converges
    to is this minimiser, which the oracle computes directly: Lawson-Hanson
    for up to 256 columns, FNNLS on the Gram form above that.
    """
    t = PhiS.shape[1]
    if t <= 256:
        return nnls_lawson_hanson(PhiS, m)
    G = PhiS.T @ PhiS
    b = PhiS.T @ m
    w0 = None
    if w_prev is not None:
        w0 = np.zeros(t)
        w0[: len(w_prev)] = w_prev
    return fnnls(G, b, w0)


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
               margin_tol: float = 1e-6) -> Selection:
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
                if margin > margin_tol:
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


def compact(Q, K, V, t, k=1, R=1, beta_in=None, scale=None, shift=None, replay=None,
            margin_tol=1e-6) -> Compaction:
    """Compact one head's (K, V) to t keys: C_k (a subset of K), per-key bias
    beta and fitted values C_v (p2 section 2; p3 pipeline)."""
    K = np.asarray(K, dtype=np.float64)
    feats = mass_features(Q, K, V, beta_in, scale, shift)
    sel = omp_select(feats.Phi, feats.m, t, k, R, replay, margin_tol)
    S = np.asarray(sel.S, dtype=np.int64)
    Cv = ols_values(feats.Phi[:, S], sel.w, feats.Y)
    beta = log_weights(sel.w)
    if beta_in is not None:
        beta = beta + np.asarray(beta_in, dtype=np.float64)[S]
    order = np.argsort(S, kind="stable")
    return Compaction(S[order], K[S[order]], beta[order], Cv[order], sel.w[order], sel, feats)


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
