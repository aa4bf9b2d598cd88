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


def test_fnnls_warm_start_same_minimiser():
    rng = np.random.default_rng(7)
    A = _phi_like(rng, 200, 50)
    y = A @ np.abs(rng.normal(size=50)) + 0.1 * rng.normal(size=200)
    G, b = A.T @ A, A.T @ y
    cold = oracle.fnnls(G, b)
    warm = oracle.fnnls(G, b, w0=np.abs(rng.normal(size=50)))
    assert np.linalg.norm(A @ (cold - warm)) <= 1e-9 * np.linalg.norm(y)


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
