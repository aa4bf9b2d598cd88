"""Pins of the float64 oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, invariants, brute force on tiny inputs, a library routine, or numbers
the pages print.  A few tests plant a plausible mistake in the oracle (on the
CPU) and show that a pin catches it.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import amc_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small_head(seed=0, n=64, T=96, d=16, outliers=False):
    return synth.make_head(seed, n, T, d, outliers, "f32")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[k] = float(v)
    return out


# ----------------------------------------------------------------------------
# attention, mass and the mixing identity
# ----------------------------------------------------------------------------
def test_attention_matches_explicit_softmax():
    rng = np.random.default_rng(1)
    Q = rng.normal(size=(5, 4))
    K = rng.normal(size=(7, 4))
    V = rng.normal(size=(7, 3))
    b = rng.normal(size=7)
    Ov, logM = oracle.attention(Q, K, V, b, scale=0.5)
    for i in range(5):
        lg = [0.5 * sum(Q[i, c] * K[j, c] for c in range(4)) + b[j] for j in range(7)]
        e = [math.exp(x) for x in lg]
        Z = sum(e)
        assert abs(math.log(Z) - logM[i]) < 1e-12
        for c in range(3):
            assert abs(sum(e[j] * V[j, c] for j in range(7)) / Z - Ov[i, c]) < 1e-12


def test_mixing_identity_random_blocks():
    rng = np.random.default_rng(2)
    for trial in range(20):
        d = 8
        Q = rng.normal(size=(10, d))
        K1, K2 = rng.normal(size=(13, d)) * 2, rng.normal(size=(9, d)) * 2
        V1, V2 = rng.normal(size=(13, 5)), rng.normal(size=(9, 5))
        b1, b2 = rng.normal(size=13) * 3, rng.normal(size=9) * 3
        O1, M1 = oracle.attention(Q, K1, V1, b1)
        O2, M2 = oracle.attention(Q, K2, V2, b2)
        Ocat, Mcat = oracle.attention(Q, np.vstack([K1, K2]), np.vstack([V1, V2]), np.concatenate([b1, b2]))
        Omix, Mmix = oracle.mix_blocks(O1, M1, O2, M2)
        assert np.max(np.abs(Ocat - Omix)) < 1e-12
        assert np.max(np.abs(Mcat - Mmix)) < 1e-12


def test_compacted_block_with_random_suffix():
    """O_cat_hat - O_cat = a_hat*delta + (a_hat - a)(O1 - O2) per query, where a
    and a_hat are the prefix's mass shares and delta the local output error."""
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    Qs, K2, V2 = synth.fresh_tokens([0, 7], h.centres, 0, 512, False, "f32")
    Q = h.Q
    O1, M1 = oracle.attention(Q, h.K, h.V)
    O1h, M1h = oracle.attention(Q, res.Ck, res.Cv, res.beta)
    O2, M2 = oracle.attention(Q, K2, V2)
    Ocat, _ = oracle.attention(Q, np.vstack([h.K, K2]), np.vstack([h.V, V2]))
    Ocat_h, _ = oracle.attention(Q, np.vstack([res.Ck, K2]), np.vstack([res.Cv, V2]),
                                 np.concatenate([res.beta, np.zeros(512)]))
    a = 1.0 / (1.0 + np.exp(M2 - M1))
    ah = 1.0 / (1.0 + np.exp(M2 - M1h))
    rhs = ah[:, None] * (O1h - O1) + (ah - a)[:, None] * (O1 - O2)
    assert np.max(np.abs((Ocat_h - Ocat) - rhs)) < 1e-10


def test_mass_features_definition():
    h = _small_head(3)
    f = oracle.mass_features(h.Q, h.K, h.V)
    sc = 1 / math.sqrt(h.Q.shape[1])
    i, j = 5, 17
    lg = sc * float(np.dot(h.Q[i], h.K[j]))
    L = sc * h.Q @ h.K.T
    assert abs(f.shift - L.max()) < 1e-12
    assert abs(f.Phi[i, j] - math.exp(lg - f.shift)) < 1e-14
    O, logM = oracle.attention(h.Q, h.K, h.V)
    assert np.allclose(np.log(f.m) + f.shift, logM, rtol=0, atol=1e-12)
    assert np.allclose(f.Y, O, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# NNLS
# ----------------------------------------------------------------------------
def _phi_like(rng, n, t, spread=6.0):
    """Columns shaped like mass features: exp of correlated logits."""
    d = 8
    Qm = rng.normal(size=(n, d))
    Km = rng.normal(size=(t, d)) * spread / math.sqrt(d)
    return np.exp(Qm @ Km.T - 2.0)


def test_nnls_t1_closed_form():
    rng = np.random.default_rng(4)
    for _ in range(50):
        phi = rng.normal(size=30)
        m = rng.normal(size=30)
        w = oracle.nnls_exact(phi[:, None], m)
        assert abs(w[0] - max(0.0, phi @ m) / (phi @ phi)) < 1e-12 * max(1, abs(w[0]))


def test_nnls_kkt_holds_on_selection():
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    S = res.selection.S
    P = res.features.Phi[:, S]
    G, b = P.T @ P, P.T @ res.features.m
    assert O.nnls_kkt_violation(G, b, res.selection.w) < 1e-8


@pytest.mark.parametrize("t", [1, 3, 8, 20, 40, 64])
def test_fnnls_matches_lawson_hanson(t):
    rng = np.random.default_rng(100 + t)
    for _ in range(5):
        A = _phi_like(rng, 128, t)
        y = A @ (np.abs(rng.normal(size=t)) * (rng.random(t) > 0.3)) + 0.05 * rng.normal(size=128) * A.mean()
        w_lh = oracle.nnls_lawson_hanson(A, y)
        w_f = oracle.fnnls(A.T @ A, A.T @ y)
        G, b = A.T @ A, A.T @ y
        assert O.nnls_kkt_violation(G, b, w_f) < 1e-8
        assert O.nnls_kkt_violation(G, b, w_lh) < 1e-8
        # same minimiser: compare the fitted vectors (well conditioned) and the weights
        assert np.linalg.norm(A @ (w_f - w_lh)) <= 1e-9 * np.linalg.norm(y)
        big = w_lh > 1e-6 * w_lh.max()
        assert np.allclose(w_f[big], w_lh[big], rtol=1e-5)


def test_fnnls_at_large_budget_well_conditioned():
    """fnnls at t = 300 on a well-conditioned system (independent Gaussian
    columns): KKT, and the minimiser of scipy's Lawson-Hanson."""
    rng = np.random.default_rng(301)
    n, t = 900, 300
    A = rng.normal(size=(n, t))
    y = A @ (np.abs(rng.normal(size=t)) * (rng.random(t) > 0.4)) + 0.3 * rng.normal(size=n)
    G, b = A.T @ A, A.T @ y
    w_f = oracle.fnnls(G, b)
    w_lh = oracle.nnls_lawson_hanson(A, y)
    assert O.nnls_kkt_violation(G, b, w_f) < 1e-8
    assert np.linalg.norm(A @ (w_f - w_lh)) <= 1e-9 * np.linalg.norm(y)
    assert np.array_equal(w_f > 0, w_lh > 0)
    big = w_lh > 1e-6 * w_lh.max()
    assert np.allclose(w_f[big], w_lh[big], rtol=1e-8)


def test_fnnls_warm_start_same_minimiser():
    rng = np.random.default_rng(7)
    A = _phi_like(rng, 200, 50)
    y = A @ np.abs(rng.normal(size=50)) + 0.1 * rng.normal(size=200)
    G, b = A.T @ A, A.T @ y
    cold = oracle.fnnls(G, b)
    warm = oracle.fnnls(G, b, w0=np.abs(rng.normal(size=50)))
    assert np.linalg.norm(A @ (cold - warm)) <= 1e-9 * np.linalg.norm(y)


def _collinear_selection(t=40):
    """A nearly collinear selection with an almost exact mass fit: 40 keys of
    plain OMP on a 300-query, 700-key head (d = 64), where cond(Phi_S) reaches
    1e8 and the relative residual 6e-10.  Gram-form solvers lose this regime
    (the Gram matrix's conditioning is the square of Phi_S's)."""
    h = synth.make_head([34, 0], 300, 700, 64, True, "bf16")
    b = synth.random_beta([35, 0], 700, 1.0)
    f = oracle.mass_features(h.Q, h.K, h.V, b)
    sel = O.omp_select(f.Phi, f.m, t)
    return f.Phi[:, sel.S], f.m


def _objective(A, y, w):
    """||A w - y|| in extended precision (the objective, free of the rounding
    of the fp64 evaluation)."""
    r = np.asarray(y, dtype=np.longdouble) - np.asarray(A, dtype=np.longdouble) @ np.asarray(w, dtype=np.longdouble)
    return float(np.sqrt(np.sum(r * r)))


@pytest.mark.parametrize("t", [5, 40, 120])
def test_nnls_qr_matches_lawson_hanson(t):
    """The QR-reduced active-set solver and scipy's Lawson-Hanson on Phi_S
    reach the same minimiser on well-conditioned systems."""
    rng = np.random.default_rng(300 + t)
    for _ in range(3):
        A = _phi_like(rng, 2 * t + 50, t)
        y = A @ (np.abs(rng.normal(size=t)) * (rng.random(t) > 0.3)) + 0.05 * rng.normal(size=2 * t + 50) * A.mean()
        w_lh = oracle.nnls_lawson_hanson(A, y)
        w_qr = oracle.nnls_qr(A, y)
        assert abs(_objective(A, y, w_qr) / _objective(A, y, w_lh) - 1) < 1e-12
        big = w_lh > 1e-6 * w_lh.max()
        assert np.allclose(w_qr[big], w_lh[big], rtol=1e-6)
        assert np.all(w_qr[~big] <= 1e-6 * w_lh.max())


def test_nnls_qr_large_selection_matches_lawson_hanson():
    """Above 256 keys the oracle's refit is nnls_qr: at t = 300 on a real
    selection (512 queries) it agrees with Lawson-Hanson on Phi_S, which the
    Gram-form FNNLS does not do there."""
    h = synth.make_head([36, 0], 512, 1024, 128, True, "bf16")
    f = oracle.mass_features(h.Q, h.K, h.V)
    sel = O.omp_select(f.Phi, f.m, 300, 4, 2)
    P = f.Phi[:, sel.S]
    w_lh = oracle.nnls_lawson_hanson(P, f.m)
    w_qr = oracle.nnls_exact(P, f.m)
    ob_lh, ob_qr = _objective(P, f.m, w_lh), _objective(P, f.m, w_qr)
    assert abs(ob_qr / ob_lh - 1) < 1e-10
    both = (w_lh > 0) & (w_qr > 0)
    assert np.max(np.abs(np.log(w_lh[both]) - np.log(w_qr[both]))) < 1e-6
    assert np.array_equal(w_lh > 0, w_qr > 0)


def test_nnls_qr_extended_precision_on_collinear_selection():
    """On the nearly collinear selection the float64 solve reaches the minimum
    that the same method finds in extended precision (objective to 1e-10,
    beta to 1e-6), and so does Lawson-Hanson; a gradient-threshold test on the
    Gram form stops well above it."""
    P, m = _collinear_selection()
    w64 = oracle.nnls_qr(P, m)
    wld = oracle.nnls_qr(P, m, dtype=np.longdouble)
    w_lh = oracle.nnls_lawson_hanson(P, m)
    ob = _objective(P, m, wld)
    assert abs(_objective(P, m, w64) / ob - 1) < 1e-10
    assert abs(_objective(P, m, w_lh) / ob - 1) < 1e-10
    both = (w64 > 0) & (wld > 0)
    assert np.array_equal(w64 > 0, wld > 0)
    assert np.max(np.abs(np.log(w64[both]) - np.log(wld[both]))) < 1e-6
    # the Gram form: its KKT point is not the minimiser here
    w_g = oracle.fnnls(P.T @ P, P.T @ m)
    assert _objective(P, m, w_g) / ob - 1 > 1e-3


def test_nnls_qr_warm_start_same_minimiser():
    P, m = _collinear_selection(32)
    cold = oracle.nnls_qr(P, m)
    rng = np.random.default_rng(9)
    warm = oracle.nnls_qr(P, m, w0=np.abs(rng.normal(size=P.shape[1])) * (rng.random(P.shape[1]) > 0.5))
    assert abs(_objective(P, m, warm) / _objective(P, m, cold) - 1) < 1e-10
    assert np.array_equal(cold > 0, warm > 0)


def test_nnls_lh_update_follows_nnls_qr():
    """The updating form of the Lawson-Hanson iteration against the
    refactoring one, on systems with dependent columns, fewer rows than
    columns, zero columns and warm starts: the same minimum (1e-9 of |m|) and,
    on full-rank systems, the same weights."""
    rng = np.random.default_rng(44)
    for trial in range(120):
        n = int(rng.integers(2, 50))
        t = int(rng.integers(1, 40))
        A = np.abs(rng.normal(size=(n, t))) ** rng.uniform(0.5, 3)
        if trial % 4 == 0 and t > 3:
            A[:, 2] = 0.5 * (A[:, 0] + A[:, 1])
        if trial % 9 == 0 and t > 1:
            A[:, 1] = 0.0
        m = A @ (np.abs(rng.normal(size=t)) * (rng.random(t) > 0.3)) + np.abs(rng.normal(size=n)) * rng.uniform(0, 1)
        w_qr = oracle.nnls_qr(A, m)
        w0 = None if trial % 3 else w_qr * rng.uniform(0.2, 2.0, size=t) * (rng.random(t) > 0.4)
        w_up = oracle.nnls_lh_update(A, m, w0=w0)
        assert np.all(w_up >= 0)
        nm = np.linalg.norm(m)
        assert abs(_objective(A, m, w_up) - _objective(A, m, w_qr)) <= 1e-9 * nm
        if n >= t + 5 and trial % 4 and trial % 9:
            assert np.allclose(w_up, w_qr, rtol=1e-7, atol=1e-9 * w_qr.max(initial=1.0))


def test_nnls_lh_update_kkt_at_large_budget():
    """At t = 1000 of a real head (2048 queries) the updating solver reaches
    a KKT point of the refit (violation below 1e-10, a hundredth of what
    nnls_exact accepts from scipy; the stall stop ends it once 64 entering
    steps gain less than 1e-15 of |m|), and agrees with the refactoring
    solver's minimum at t = 300 on the same head."""
    h = synth.make_head([45, 0], 2048, 4096, 128, True, "bf16")
    f = oracle.mass_features(h.Q, h.K, h.V)
    order = np.argsort(-O.highest_scores(f.Phi, f.m), kind="stable")
    P = f.Phi[:, order[:1000]]
    w = oracle.nnls_lh_update(P, f.m)
    assert O.nnls_kkt_violation(P.T @ P, P.T @ f.m, w) < 1e-10
    P3 = f.Phi[:, order[:300]]
    w3, q3 = oracle.nnls_lh_update(P3, f.m), oracle.nnls_qr(P3, f.m)
    assert abs(_objective(P3, f.m, w3) / _objective(P3, f.m, q3) - 1) < 1e-9
    both = (w3 > 0) & (q3 > 0)
    assert np.array_equal(w3 > 0, q3 > 0)
    assert np.max(np.abs(np.log(w3[both]) - np.log(q3[both]))) < 1e-6


def test_nnls_iteration_caps_raise():
    """An exhausted iteration cap is an error, not a silent return."""
    rng = np.random.default_rng(12)
    A = _phi_like(rng, 80, 30)
    y = A @ np.abs(rng.normal(size=30))
    with pytest.raises(RuntimeError):
        oracle.fnnls(A.T @ A, A.T @ y, max_outer=2)
    with pytest.raises(RuntimeError):
        oracle.nnls_qr(A, y, max_outer=2)
    with pytest.raises(RuntimeError):
        oracle.nnls_lh_update(A, y, max_outer=2)


def test_planted_coarse_dependence_test_misses_minimiser(monkeypatch):
    """Planted mistake: a dependence threshold of 1e-6 on the complement norm
    (unit columns) rejects keys the minimiser needs on the collinear
    selection (their complement norms lie near 1e-7); the objective rises far
    above the extended-precision minimum the pin above compares against."""
    P, m = _collinear_selection()
    good = _objective(P, m, oracle.nnls_qr(P, m))
    monkeypatch.setattr(O, "DEP_TOL", 1e-6)
    bad = _objective(P, m, oracle.nnls_qr(P, m))
    assert bad / good - 1 > 1e-3


def test_score_tie_bound_covers_float64_spread():
    """The replay's tie bound (score_tie_ulps) against what float64 actually
    resolves.  On the collinear selection, two exact solvers (Lawson-Hanson
    and nnls_qr, equal objectives to 1e-12) give scores whose spread on the
    top two keys reaches their gap (at 38 keys they even order them
    differently): the bound covers that spread.  At 30 keys the scores are
    resolved, and the bound is far below the gap."""
    h = synth.make_head([34, 0], 300, 700, 64, True, "bf16")
    b = synth.random_beta([35, 0], 700, 1.0)
    f = oracle.mass_features(h.Q, h.K, h.V, b)
    sel = O.omp_select(f.Phi, f.m, 40)
    eb = O.score_tie_ulps(h.Q, h.K, 40, b) * np.finfo(np.float64).eps
    bj = f.Phi.T @ f.m
    for it, resolved in ((30, True), (32, False), (36, False), (38, False)):
        S = sel.S[:it]
        P = f.Phi[:, S]
        c1 = f.Phi.T @ (f.m - P @ oracle.nnls_lawson_hanson(P, f.m))
        c2 = f.Phi.T @ (f.m - P @ oracle.nnls_qr(P, f.m))
        c1[S] = c2[S] = -np.inf
        top = np.argsort(-c1)[:2]
        bound = eb * (bj[top[0]] + bj[top[1]])
        gap = c1[top[0]] - c1[top[1]]
        spread = np.max(np.abs(c1[top] - c2[top]))
        assert spread <= bound
        if resolved:
            assert bound < 1e-6 * gap
        else:
            assert gap < bound


def test_replay_flags_a_resolved_swap():
    """Planted mistake in a replayed selection: at iteration 5 of workload 0
    the replay takes the oracle's second-best key.  The scores are resolved
    there, so the replay reports a mismatch (the tie bound does not hide it)."""
    h = synth.workload(0).head(0)
    ref = oracle.compact(h.Q, h.K, h.V, 12)
    f = ref.features
    picks = [[j] for j in ref.selection.S]
    S4 = ref.selection.S[:4]
    w = oracle.nnls_exact(f.Phi[:, S4], f.m)
    c = f.Phi.T @ (f.m - f.Phi[:, S4] @ w)
    c[S4] = -np.inf
    second = int(np.argsort(-c)[1])
    bad = picks[:4] + [[second]] + [[j] for j in ref.selection.S[4:] if j != second][:7]
    rep = oracle.compact(h.Q, h.K, h.V, 12, replay=bad)
    assert rep.selection.steps[4].mismatch


def test_errors_hand_computed():
    """errors() on a case worked by hand: d = 1 (scale 1), keys 0 and log 3
    with values 1 and 2; queries 1 and 0.  Original masses (4, 2), outputs
    (7/4, 3/2).  Compacted to key 0 with beta = log 2 and value 1: masses
    (2, 2), outputs (1, 1)."""
    Q = np.array([[1.0], [0.0]])
    K = np.array([[0.0], [math.log(3.0)]])
    V = np.array([[1.0], [2.0]])
    e_mass, e_out = oracle.errors(Q, K, V, np.array([[0.0]]), np.array([math.log(2.0)]), np.array([[1.0]]))
    assert abs(e_mass - math.sqrt(4.0) / math.sqrt(20.0)) < 1e-14
    assert abs(e_out - math.sqrt(0.75 ** 2 + 0.5 ** 2) / math.sqrt(1.75 ** 2 + 1.5 ** 2)) < 1e-14


# ----------------------------------------------------------------------------
# closed form: budget t = T
# ----------------------------------------------------------------------------
def test_full_budget_is_identity():
    """With t = T and n >= T the fit is exact: w = 1, beta = 0, C_v = V and both
    errors vanish."""
    h = synth.make_head(np.random.SeedSequence([0, 5]), 256, 64, 64, False, "f32")
    res = oracle.compact(h.Q, h.K, h.V, 64)
    assert np.array_equal(res.sel_idx, np.arange(64))
    assert np.max(np.abs(res.w - 1.0)) < 1e-7
    assert np.max(np.abs(res.beta)) < 1e-7
    assert np.max(np.abs(res.Cv - h.V)) < 1e-6
    e_mass, e_out = oracle.errors(h.Q, h.K, h.V, res.Ck, res.beta, res.Cv)
    assert e_mass < 1e-9 and e_out < 1e-9


# ----------------------------------------------------------------------------
# brute force on tiny inputs
# ----------------------------------------------------------------------------
def _bf_phi(Q, K):
    """exp(q.k / sqrt(d) - s), written out with explicit loops."""
    n, d = Q.shape
    T = K.shape[0]
    sc = 1.0 / math.sqrt(d)
    L = [[sc * sum(Q[i, c] * K[j, c] for c in range(d)) for j in range(T)] for i in range(n)]
    s = max(max(row) for row in L)
    return np.array([[math.exp(x - s) for x in row] for row in L])


def _bf_nnls(A, y):
    """Exact NNLS by enumerating every support: the minimiser is the least
    squares solution on its support, and it is feasible."""
    t = A.shape[1]
    best, best_w = math.inf, np.zeros(t)
    for mask in range(1 << t):
        P = [j for j in range(t) if (mask >> j) & 1]
        w = np.zeros(t)
        if P:
            sol = np.linalg.lstsq(A[:, P], y, rcond=None)[0]
            if np.any(sol < 0):
                continue
            w[P] = sol
        res = float(np.linalg.norm(A @ w - y))
        if res < best - 1e-15:
            best, best_w = res, w
    return best_w, best


def _bf_greedy(Phi, m, t):
    n, T = Phi.shape
    S, r = [], m.copy()
    w = np.zeros(0)
    for _ in range(t):
        best_j, best_c = None, -math.inf
        for j in range(T):
            if j in S:
                continue
            c = sum(r[i] * Phi[i, j] for i in range(n))
            if c > best_c:
                best_j, best_c = j, c
        S.append(best_j)
        w, _ = _bf_nnls(Phi[:, S], m)
        r = np.array([m[i] - sum(Phi[i, S[a]] * w[a] for a in range(len(S))) for i in range(n)])
    return S, w, r


def test_brute_force_greedy_trajectory():
    """On T <= 10, t <= 2 the oracle's selection and weights equal an explicit
    enumeration of every candidate at every step and every NNLS support."""
    attained = {1: 0, 2: 0}
    for seed in range(300):
        rng = np.random.default_rng(seed)
        T = int(rng.integers(3, 11))
        h = synth.make_head([11, seed], 16, T, 8, False, "f32")
        Phi = _bf_phi(h.Q, h.K)
        m = Phi.sum(axis=1)
        f = oracle.mass_features(h.Q, h.K, h.V)
        assert np.max(np.abs(f.Phi - Phi)) < 1e-13
        for t in (1, 2):
            S, w, r = _bf_greedy(Phi, m, t)
            sel = oracle.omp_select(f.Phi, f.m, t)
            assert sel.S == S, (seed, t)
            PS = Phi[:, S]
            assert np.linalg.norm(PS @ (sel.w - w)) <= 1e-12 * np.linalg.norm(m)
            cond = np.linalg.cond(PS)
            assert np.allclose(sel.w, w, rtol=1e-13 * cond + 1e-12, atol=1e-12)
            # best subset can only do better than greedy
            omp_res = float(np.linalg.norm(r))
            best = min(_bf_nnls(Phi[:, list(c)], m)[1] for c in itertools.combinations(range(T), t))
            assert best <= omp_res * (1 + 1e-12) + 1e-15
            attained[t] += best >= omp_res * (1 - 1e-9)
    # greedy is not best-subset in general; record that it usually is
    assert attained[1] > 150 and attained[2] > 100


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_shift_invariance():
    h = synth.workload(0).head(0)
    base = oracle.compact(h.Q, h.K, h.V, 32)
    s = base.features.shift
    for delta in (-5.0, 5.0):
        other = oracle.compact(h.Q, h.K, h.V, 32, shift=s + delta)
        assert np.array_equal(other.sel_idx, base.sel_idx)
        fin = np.isfinite(base.beta)
        assert np.array_equal(fin, np.isfinite(other.beta))
        assert np.max(np.abs(other.beta[fin] - base.beta[fin])) < 1e-8
        assert np.max(np.abs(other.Cv - base.Cv)) < 1e-6 * np.max(np.abs(base.Cv))


def test_residual_monotone_and_mass_error_monotone_in_budget():
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    norms = [st.resid_norm for st in res.selection.steps if st.refit]
    assert all(b <= a * (1 + 1e-10) for a, b in zip(norms, norms[1:]))
    prev = math.inf
    for t in (2, 4, 8, 16, 32):
        r = oracle.compact(h.Q, h.K, h.V, t)
        e_mass, _ = oracle.errors(h.Q, h.K, h.V, r.Ck, r.beta, r.Cv)
        assert e_mass <= prev * (1 + 1e-9)
        prev = e_mass


def test_batched_selection_readings():
    """k = R = 1 is plain OMP; with a stale residual between refits, (k, R) and
    (k*R, 1) select the same keys."""
    h = synth.workload(0).head(0)
    f = oracle.mass_features(h.Q, h.K, h.V)
    plain = oracle.omp_select(f.Phi, f.m, 32)
    one = oracle.omp_select(f.Phi, f.m, 32, k=1, R=1)
    assert plain.S == one.S
    a = oracle.omp_select(f.Phi, f.m, 30, k=4, R=2)
    b = oracle.omp_select(f.Phi, f.m, 30, k=8, R=1)
    assert set(a.S) == set(b.S)
    assert np.allclose(np.sort(a.w), np.sort(b.w), rtol=1e-9, atol=0)
    sizes = O.iteration_sizes(30, 4, 2)
    assert [s for s, _ in sizes] == [4] * 7 + [2]
    assert [rf for _, rf in sizes] == [False, True] * 3 + [False, True]


def test_bias_in_equals_duplicate_key():
    """A key carrying beta_in = log 2 contributes exactly like two copies."""
    h = _small_head(5)
    j = 11
    b = np.zeros(h.K.shape[0])
    b[j] = math.log(2.0)
    f1 = oracle.mass_features(h.Q, h.K, h.V, bias=b)
    K2 = np.vstack([h.K, h.K[j:j + 1]])
    V2 = np.vstack([h.V, h.V[j:j + 1]])
    f2 = oracle.mass_features(h.Q, K2, V2, shift=f1.shift)
    assert np.allclose(f1.m, f2.m, rtol=1e-12, atol=0)
    assert np.allclose(f1.Y, f2.Y, rtol=0, atol=1e-12)
    assert np.allclose(f1.Phi[:, j], f2.Phi[:, j] + f2.Phi[:, -1], rtol=1e-12)
    zero = oracle.compact(h.Q, h.K, h.V, 12, beta_in=np.zeros(h.K.shape[0]))
    plain = oracle.compact(h.Q, h.K, h.V, 12)
    assert np.array_equal(zero.sel_idx, plain.sel_idx)
    assert np.allclose(zero.beta, plain.beta, rtol=0, atol=0)


def test_permutation_of_keys():
    h = _small_head(6, n=80, T=120)
    base = oracle.compact(h.Q, h.K, h.V, 10)
    perm = np.random.default_rng(6).permutation(120)
    other = oracle.compact(h.Q, h.K[perm], h.V[perm], 10)
    assert set(perm[other.sel_idx].tolist()) == set(base.sel_idx.tolist())


def test_ols_is_optimal_for_the_attention_output():
    """The value fit minimises the compacted block's attention-output error
    as computed by the independent softmax evaluator: the gradient of
    ||softmax(Q Ck^T/sqrt(d) + beta) Cv - O||^2 in Cv vanishes."""
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    O_ref, _ = oracle.attention(h.Q, h.K, h.V)
    L = oracle.logits(h.Q, res.Ck, res.beta)
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    Oc = P @ res.Cv
    grad = P.T @ (Oc - O_ref)
    assert np.max(np.abs(grad)) < 1e-9 * np.max(np.abs(P.T @ O_ref))
    # linear in V
    V2 = np.random.default_rng(9).normal(size=h.V.shape)
    feats1 = oracle.mass_features(h.Q, h.K, h.V)
    feats2 = oracle.mass_features(h.Q, h.K, V2)
    S = res.selection.S
    c1 = oracle.ols_values(feats1.Phi[:, S], res.selection.w, feats1.Y)
    c2 = oracle.ols_values(feats1.Phi[:, S], res.selection.w, feats2.Y)
    c3 = oracle.ols_values(feats1.Phi[:, S], res.selection.w, feats1.Y * 2.5 + feats2.Y)
    assert np.allclose(c3, 2.5 * c1 + c2, rtol=0, atol=1e-8 * np.max(np.abs(c3)))


def test_beta_reproduces_fitted_mass():
    """With beta = log w the compacted block's mass, evaluated by the softmax
    evaluator, is Phi_S w (times e^s), the NNLS fit of the target mass."""
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    S = res.selection.S
    mhat = res.features.Phi[:, S] @ res.selection.w
    _, logMc = oracle.attention(h.Q, res.Ck, res.Cv, res.beta)
    assert np.allclose(np.exp(logMc - res.features.shift), mhat, rtol=1e-12)


def test_zero_weight_key_is_masked():
    h = synth.workload(0).head(0)
    res = oracle.compact(h.Q, h.K, h.V, 32)
    dead = res.w == 0
    assert dead.sum() >= 1
    assert np.all(np.isneginf(res.beta[dead]))
    assert np.all(res.Cv[dead] == 0)


# ----------------------------------------------------------------------------
# replay protocol
# ----------------------------------------------------------------------------
def test_replay_of_own_picks_is_clean_and_wrong_pick_is_caught():
    h = synth.workload(0).head(0)
    f = oracle.mass_features(h.Q, h.K, h.V)
    sel = oracle.omp_select(f.Phi, f.m, 16)
    picks = [st.picks for st in sel.steps]
    again = oracle.omp_select(f.Phi, f.m, 16, replay=picks)
    assert not any(st.mismatch or st.forced for st in again.steps)
    bad = [list(p) for p in picks]
    c = f.Phi.T @ f.m
    worst = int(np.argmin(c))
    bad[0] = [worst]
    caught = oracle.omp_select(f.Phi, f.m, 16, replay=bad)
    assert caught.steps[0].mismatch


# ----------------------------------------------------------------------------
# numbers the pages print
# ----------------------------------------------------------------------------
def test_golden_overhead_factor():
    g = _read_golden("overhead.txt")
    d = int(g["head_dim"])
    h = synth.make_head([3, 3], 300, 200, d, True, "bf16")
    res = oracle.compact(h.Q, h.K, h.V, 4)
    per_token = res.Ck.shape[1] + res.Cv.shape[1] + 1  # key + value + one bias
    assert res.beta.shape == (4,)
    assert per_token * g["denominator"] == g["numerator"] * (2 * d)


def test_golden_online_schedule():
    g = _read_golden("online_schedule.txt")
    eff = O.online_effective_length(int(g["physical"]), int(g["keep_newest"]), int(g["rounds"]), g["ratio"])
    assert eff == 2048 + 6 * 1014
    assert abs(eff - g["effective_reported"]) / g["effective_reported"] < 0.01


# ----------------------------------------------------------------------------
# planted mistakes are caught by the pins above
# ----------------------------------------------------------------------------
def test_planted_unconstrained_fit_breaks_kkt(monkeypatch):
    monkeypatch.setattr(O, "nnls_exact", lambda P, m, w_prev=None: np.linalg.lstsq(P, m, rcond=None)[0])
    h = synth.workload(0).head(0)
    f = oracle.mass_features(h.Q, h.K, h.V)
    sel = O.omp_select(f.Phi, f.m, 32)
    P = f.Phi[:, sel.S]
    assert O.nnls_kkt_violation(P.T @ P, P.T @ f.m, sel.w) > 1e-6


def test_planted_missing_normaliser_breaks_ols_optimality(monkeypatch):
    def bad_ols(PhiS, w, Y):
        F = w > 0
        A = PhiS[:, F] * w[F][None, :]  # forgot the 1/mhat row weights
        Cv = np.zeros((w.shape[0], Y.shape[1]))
        Cv[F] = np.linalg.lstsq(A, Y, rcond=None)[0]
        return Cv

    monkeypatch.setattr(O, "ols_values", bad_ols)
    h = synth.workload(0).head(0)
    res = O.compact(h.Q, h.K, h.V, 32)
    O_ref, _ = oracle.attention(h.Q, h.K, h.V)
    L = oracle.logits(h.Q, res.Ck, res.beta)
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    grad = P.T @ (P @ res.Cv - O_ref)
    assert np.max(np.abs(grad)) > 1e-6 * np.max(np.abs(P.T @ O_ref))


def test_planted_stale_residual_breaks_brute_force(monkeypatch):
    real = O.omp_select

    def never_update(Phi, m, t, k=1, R=1, replay=None, margin_tol=1e-6):
        # scores every step against m instead of the residual
        sel = real(Phi, m, 1)
        c = Phi.T @ m
        order = np.lexsort((np.arange(c.shape[0]), -c))
        S = [int(j) for j in order[:t]]
        return O.Selection(S, O.nnls_exact(Phi[:, S], m), m - Phi[:, S] @ O.nnls_exact(Phi[:, S], m), sel.steps)

    monkeypatch.setattr(O, "omp_select", never_update)
    differs = 0
    for seed in range(60):
        rng = np.random.default_rng(seed)
        T = int(rng.integers(3, 11))
        h = synth.make_head([11, seed], 16, T, 8, False, "f32")
        Phi = _bf_phi(h.Q, h.K)
        S, _, _ = _bf_greedy(Phi, Phi.sum(axis=1), 2)
        f = oracle.mass_features(h.Q, h.K, h.V)
        differs += O.omp_select(f.Phi, f.m, 2).S != S
    assert differs > 0


# ----------------------------------------------------------------------------
# AM-Highest (p3 "Method Family and Trade-offs"; p4, highest-attention keys)
# ----------------------------------------------------------------------------
def _softmax_scores_by_loops(Q, K, bias, scale):
    """Each key's attention summed over the queries, one query's softmax at a time."""
    n, T = Q.shape[0], K.shape[0]
    score = [0.0] * T
    for i in range(n):
        logits = []
        for j in range(T):
            dot = 0.0
            for c in range(Q.shape[1]):
                dot += float(Q[i, c]) * float(K[j, c])
            logits.append(scale * dot + (0.0 if bias is None else float(bias[j])))
        mx = max(logits)
        ex = [math.exp(v - mx) for v in logits]
        tot = sum(ex)
        for j in range(T):
            score[j] += ex[j] / tot
    return np.array(score)


def test_highest_matches_brute_force_softmax():
    rng = np.random.default_rng(410)
    for trial in range(40):
        n, T, d = int(rng.integers(1, 6)), int(rng.integers(3, 10)), 4
        t = int(rng.integers(1, T + 1))
        Q, K = rng.normal(size=(n, d)), rng.normal(size=(T, d)) * 1.5
        bias = rng.normal(size=T) if trial % 2 else None
        V = rng.normal(size=(T, 3))
        ref = _softmax_scores_by_loops(Q, K, bias, 0.5)
        f = oracle.mass_features(Q, K, V, bias, 0.5)
        assert np.allclose(oracle.highest_scores(f.Phi, f.m), ref, rtol=1e-12, atol=1e-15)
        want = sorted(range(T), key=lambda j: (-ref[j], j))[:t]
        sel = oracle.highest_select(f.Phi, f.m, t)
        assert sorted(sel.S) == sorted(want)
        G, b = f.Phi[:, sel.S].T @ f.Phi[:, sel.S], f.Phi[:, sel.S].T @ f.m
        assert O.nnls_kkt_violation(G, b, sel.w) < 1e-9


def test_highest_scores_ignore_per_query_scale():
    """Dividing row i by its mass makes each query's scale irrelevant: any
    positive per-query factor (a per-query shift) leaves the scores."""
    rng = np.random.default_rng(411)
    Phi = np.exp(rng.normal(size=(30, 50)))
    m = Phi.sum(axis=1)
    D = np.exp(rng.normal(size=30) * 5.0)
    assert np.allclose(oracle.highest_scores(Phi * D[:, None], m * D), oracle.highest_scores(Phi, m), rtol=1e-13)


def test_planted_unnormalised_highest_is_caught():
    """Raw column sums of Phi (no division by the query's mass) rank the keys
    by the loudest query; the brute-force softmax pin rejects that."""
    Q = np.array([[4.0, 0.0], [0.0, 0.3], [0.0, 0.3]])
    K = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.9], [0.2, 0.2]])
    ref = _softmax_scores_by_loops(Q, K, None, 1.0)
    f = oracle.mass_features(Q, K, np.zeros((4, 1)), None, 1.0)
    raw = f.Phi.sum(axis=0)
    want = sorted(range(4), key=lambda j: (-ref[j], j))[:2]
    planted = sorted(range(4), key=lambda j: (-raw[j], j))[:2]
    assert sorted(oracle.highest_select(f.Phi, f.m, 2).S) == sorted(want)
    assert sorted(planted) != sorted(want)


def test_highest_replay_rule():
    rng = np.random.default_rng(412)
    Phi = np.exp(rng.normal(size=(40, 30)))
    m = Phi.sum(axis=1)
    sel = oracle.highest_select(Phi, m, 8)
    same = oracle.highest_select(Phi, m, 8, given=list(reversed(sel.S)))
    assert not same.steps[0].mismatch
    c = oracle.highest_scores(Phi, m)
    order = np.argsort(-c, kind="stable")
    swapped = [int(j) for j in order[:7]] + [int(order[-1])]  # the worst key instead of the 8th
    bad = oracle.highest_select(Phi, m, 8, given=swapped)
    assert bad.steps[0].mismatch


def test_nnls_exact_on_a_system_scipy_leaves_short():
    """Two queries, three keys (rank 2): scipy's Lawson-Hanson stops at a
    residual of 0.03336 with a nonzero gradient on a free variable; the
    minimiser (0.03185) is what nnls_exact returns."""
    rng = np.random.default_rng(410)
    for trial in range(17):
        n, T, d = int(rng.integers(1, 6)), int(rng.integers(3, 10)), 4
        t = int(rng.integers(1, T + 1))
        Q, K = rng.normal(size=(n, d)), rng.normal(size=(T, d)) * 1.5
        bias = rng.normal(size=T) if trial % 2 else None
        V = rng.normal(size=(T, 3))
    assert (n, T, t) == (2, 6, 3)
    f = oracle.mass_features(Q, K, V, bias, 0.5)
    A = f.Phi[:, oracle.highest_select(f.Phi, f.m, t).S]
    w_sp = oracle.nnls_lawson_hanson(A, f.m)
    w = oracle.nnls_exact(A, f.m)
    assert O.nnls_kkt_violation(A.T @ A, A.T @ f.m, w_sp) > 1e-4
    assert O.nnls_kkt_violation(A.T @ A, A.T @ f.m, w) < 1e-12
    assert np.linalg.norm(A @ w - f.m) < np.linalg.norm(A @ w_sp - f.m) - 1e-3


# ----------------------------------------------------------------------------
# KV-based chunked compaction (p2 section 3; p1 section 4.3)
# ----------------------------------------------------------------------------
def test_chunk_budgets_split():
    for T, t, L in [(1000, 100, 300), (60000, 6000, 8192), (10, 10, 3), (257, 23, 64), (7, 4, 2)]:
        split = oracle.chunk_budgets(T, t, L)
        assert split[0][0] == 0 and split[-1][1] == T
        assert all(a[1] == b[0] for a, b in zip(split, split[1:]))
        assert sum(tc for _, _, tc in split) == t
        for k0, k1, tc in split:
            assert 1 <= tc <= k1 - k0
            assert abs(tc - t * (k1 - k0) / T) < 1.0 + 1e-9 or tc == 1
    # largest remainders: 3 chunks of 3, 3, 1 keys sharing 5 -> quotas 2.14, 2.14, 0.71
    assert [tc for _, _, tc in oracle.chunk_budgets(7, 5, 3)] == [2, 2, 1]
    with pytest.raises(ValueError):
        oracle.chunk_budgets(7, 3, 2)  # four chunks, three keys


def test_chunked_full_budget_is_identity():
    """Every chunk at full budget reproduces the block exactly, so the
    concatenation does: offsets and order are right."""
    rng = np.random.default_rng(520)
    Q, K, V = rng.normal(size=(12, 8)), rng.normal(size=(20, 8)), rng.normal(size=(20, 5))
    bias = rng.normal(size=20)
    ch = oracle.compact_chunked(Q, K, V, 20, 7, beta_in=bias)
    assert np.array_equal(ch.sel_idx, np.arange(20))
    e_mass, e_out = oracle.errors(Q, K, V, ch.Ck, ch.beta, ch.Cv, bias)
    assert e_mass < 1e-12 and e_out < 1e-12


def test_chunked_concatenation_follows_the_mixing_identity():
    """Attention over the concatenated compacted chunks equals the chunks'
    own attention outputs combined by their masses."""
    rng = np.random.default_rng(521)
    Q, K, V = rng.normal(size=(30, 8)), rng.normal(size=(90, 8)) * 1.3, rng.normal(size=(90, 4))
    ch = oracle.compact_chunked(Q, K, V, 24, 30, k=2, R=2)
    O_cat, logM_cat = oracle.attention(Q, ch.Ck, ch.Cv, ch.beta)
    outs, logms = [], []
    for p in ch.chunks:
        o, lm = oracle.attention(Q, p.Ck, p.Cv, p.beta)
        outs.append(o)
        logms.append(lm)
    mx = np.max(np.stack(logms), axis=0)
    wts = [np.exp(lm - mx) for lm in logms]
    O_mix = sum(w[:, None] * o for w, o in zip(wts, outs)) / sum(wts)[:, None]
    assert np.allclose(O_cat, O_mix, rtol=1e-12, atol=1e-12)
    assert np.allclose(logM_cat, mx + np.log(sum(wts)), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# greedy-swap budget schedule (p1 section 4.2; p2 section 4)
# ----------------------------------------------------------------------------
def _best_allocation(L, units):
    H, J = L.shape
    best, arg = None, None
    for alloc in itertools.product(range(1, J + 1), repeat=H):
        if sum(alloc) != units:
            continue
        v = sum(L[h, a - 1] for h, a in enumerate(alloc))
        if best is None or v < best - 1e-15:
            best, arg = v, alloc
    return best, arg


def test_greedy_swap_reaches_brute_force_optimum_on_convex_curves():
    rng = np.random.default_rng(530)
    for trial in range(60):
        H, J = int(rng.integers(2, 5)), int(rng.integers(2, 6))
        units = int(rng.integers(H, H * J + 1))
        L = synth.sensitivity_curves([531, trial], H, J)
        b, _ = oracle.greedy_swap_budgets(L, 8, units * 8)
        assert sum(b) == units * 8 and all(8 <= x <= 8 * J for x in b)
        got = sum(L[h, b[h] // 8 - 1] for h in range(H))
        best, _ = _best_allocation(L, units)
        assert got <= best + 1e-12


def test_greedy_swap_even_and_flat_cases():
    L = np.tile(np.exp(-np.arange(1, 7) / 2.0), (4, 1))
    b, moves = oracle.greedy_swap_budgets(L, 10, 4 * 30)
    assert b == [30, 30, 30, 30] and moves == 0
    L2 = L.copy()
    L2[2] = 1.0  # a head insensitive to its budget gives all but one unit away
    b2, _ = oracle.greedy_swap_budgets(L2, 10, 4 * 30)
    assert b2[2] == 10 and sum(b2) == 120
