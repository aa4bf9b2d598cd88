"""Helpers shared by the GPU tests, the smoke check and the benchmark:
moving seeded inputs to the device, and comparing a libamc compaction with
the float64 oracle under the replay protocol.

Replay protocol: the oracle re-runs the greedy selection, following the
GPU's picks.  At each iteration where the oracle's own margin (score of the
last pick minus the best unpicked score, over the top score) exceeds 1e-6,
the GPU's picks must be the oracle's; below that the GPU's pick is accepted.
Then: beta within 1e-3 (absolute) on keys active on both sides, a key active
on one side only carries at most 1e-6 of that side's largest weight, and the
relative mass and attention-output errors of the GPU's compacted block are
within 1e-3 (absolute) of the oracle's own.

The beta rule presumes the NNLS weights are determined to that accuracy by
the float64 data.  Where the GPU's beta misses it, the check asks whether
they are: (i) the columns of the two supports together must have full
numerical rank (relative smallest singular value above NULL_SV; below it the
minimisers form a face and both weight vectors lie on it), and (ii) the same
NNLS solved again in extended precision (long double, warm-started from the
oracle's float64 minimiser; above LD_MAX_T keys, which that solve cannot
afford, the same NNLS in float64 on data moved by its own rounding, a
relative 2^-52 per entry) must not move beta past the tolerance.  Only
where one of these fails are the GPU's weights held to the minimum value
instead: their NNLS residual within 1e-6 (relative) of the oracle's, and its
errors to those of the oracle's own value fit on the GPU's weights (the value
fit depends on the point of the face).  Such heads are counted; a test fails
when more than FALLBACK_SHARE of its heads need it.

Replayed picks: the oracle's scores carry a float64 rounding bound (see
oracle.omp_select, tie_ulps); a replayed pick is a mismatch only where a key
it leaves out scores higher by more than both 1e-6 of the top score and the
two keys' bounds.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from oracle import amc_oracle as O

MARGIN_TOL = 1e-6
BETA_TOL = 1e-3
ERR_TOL = 1e-3
WEIGHT_REL = 1e-6
RESID_REL = 1e-6
FALLBACK_SHARE = 0.25  # largest share of a test's heads held to the minimum value only
LD_MAX_T = 512  # largest budget the extended-precision envelope is computed for (then: rounding-level data)
NULL_SV = 1e-10  # relative singular value below which columns count as dependent

REPORTS = []  # every replay report of the session (summarised at its end by conftest)


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(device)


def pack_heads(heads, dtype: str, device="cuda"):
    """Concatenates per-head (Q, K, V) into packed device tensors and offsets."""
    cu_q, cu_k = [0], [0]
    for h in heads:
        cu_q.append(cu_q[-1] + h.Q.shape[0])
        cu_k.append(cu_k[-1] + h.K.shape[0])
    Q = to_device(np.concatenate([h.Q for h in heads]), dtype, device)
    K = to_device(np.concatenate([h.K for h in heads]), dtype, device)
    V = to_device(np.concatenate([h.V for h in heads]), dtype, device)
    return Q, K, V, cu_q, cu_k


def head_outputs(res, h: int):
    Ck, beta, Cv, sel = res.head(h)
    return (Ck.float().cpu().numpy().astype(np.float64), beta.cpu().numpy().astype(np.float64),
            Cv.float().cpu().numpy().astype(np.float64), sel.cpu().numpy().astype(np.int64))


def replay_check(Q, K, V, t: int, k: int, R: int, res, h: int, beta_in=None, trace=None, select: str = "omp"):
    """Compares head h of a libamc result (run with trace=True) with the
    oracle.  Returns a report dict; ``report['ok']`` is the verdict.
    select "highest": AM-Highest (k, R unused); the oracle checks the GPU's
    key set against its own scores under the same margin rule."""
    if trace is None:
        trace = res.trace()
    picks_order = [int(j) for j in trace["pick"][h]]
    if select == "highest":
        ref = oracle.compact(Q, K, V, t, beta_in=beta_in, replay=picks_order, margin_tol=MARGIN_TOL,
                             select="highest")
    else:
        sizes = O.iteration_sizes(t, k, R)
        per_it, pos = [], 0
        for kk, _ in sizes:
            per_it.append(picks_order[pos: pos + kk])
            pos += kk
        ref = oracle.compact(Q, K, V, t, k, R, beta_in=beta_in, replay=per_it, margin_tol=MARGIN_TOL)
    Ck, beta, Cv, sel = head_outputs(res, h)
    rep = {"mismatch_iters": [s.it for s in ref.selection.steps if s.mismatch],
           "forced_iters": [s.it for s in ref.selection.steps if s.forced],
           "min_margin": float(min(s.margin for s in ref.selection.steps))}
    rep["same_set"] = bool(np.array_equal(np.asarray(ref.sel_idx), sel))
    rep["ck_exact"] = bool(np.array_equal(Ck, np.asarray(K, dtype=np.float64)[sel])) if rep["same_set"] else False
    P = ref.features.Phi[:, np.asarray(ref.sel_idx)]
    # the GPU's float64 weights (trace, selection order) in ascending key order
    order = np.argsort(np.asarray(trace["pick"][h]), kind="stable")
    w_gpu64 = np.asarray(trace["weight"][h], dtype=np.float64)[order]
    relres_gpu = float(trace["relres"][h][-1]) if "relres" in trace and len(trace["relres"][h]) else None
    _judge_weights(rep, Q, K, V, P, ref.features.m, ref.features.Y, ref.w, (ref.Ck, ref.beta, ref.Cv), sel, Ck,
                   beta, Cv, w_gpu64, relres_gpu, beta_in)
    rep["ok"] = (not rep["mismatch_iters"] and rep["same_set"] and rep["ck_exact"] and rep["weights_ok"] and
                 rep["e_mass_diff"] <= ERR_TOL and rep["e_out_diff"] <= ERR_TOL and rep["relres_ok"])
    rep["t"] = int(t)
    REPORTS.append(rep)
    return rep


def spot_replay(Q, K, V, t: int, k: int, R: int, res, h: int, cycles, beta_in=None, trace=None, final=True):
    """Spot replay of one large head at chosen refits (a full replay solves an
    exact NNLS at every refit, which large budgets cannot afford).  For each
    refit c in `cycles` (1-based, the refit after iteration c R or after the
    last one), the oracle takes the GPU's keys through that refit, solves the
    exact NNLS on them (oracle.nnls_exact, cold), scores every other key by
    Phi^T r and replays the iterations up to the next refit, all on that
    residual, under the replay rule (a mismatch needs a key left out to score
    above a key taken by more than 1e-6 of the top score and by more than the
    two keys' float64 bounds).  Beside it: the relative residual of the GPU's
    own refit c (its trace) and the minimum's.  final: after the last refit,
    the weights and errors on the GPU's key set as in replay_check.  Returns
    a report; report['ok'] is the verdict."""
    if trace is None:
        trace = res.trace()
    picks = [int(j) for j in trace["pick"][h]]
    feats = O.mass_features(Q, K, V, beta_in)
    Phi, m = feats.Phi, feats.m
    T = Phi.shape[1]
    nm = float(np.linalg.norm(m))
    eb = O.score_tie_ulps(Q, K, t, beta_in) * np.finfo(np.float64).eps
    b_all = np.abs(Phi).T @ np.abs(m)
    sizes = O.iteration_sizes(t, k, R)
    refit_at, pos = [], 0
    for i, (kk, refit) in enumerate(sizes):
        pos += kk
        if refit:
            refit_at.append((pos, i + 1))  # keys through the refit, index of the next iteration
    relres_tr = trace["relres"][h] if "relres" in trace else []
    rep = {"t": int(t), "cycles": {}, "mismatch_iters": [], "forced_iters": []}
    for c in cycles:
        p, it = refit_at[c - 1]
        PS = Phi[:, picks[:p]]
        w = O.nnls_exact(PS, m)
        r = m - PS @ w
        cyc = {"keys": p, "relres_min": float(np.linalg.norm(r)) / nm}
        if c - 1 < len(relres_tr):
            cyc["relres_gpu"] = float(relres_tr[c - 1])
        sc = Phi.T @ r
        selected = np.zeros(T, dtype=bool)
        selected[picks[:p]] = True
        pos = p
        while it < len(sizes):
            kk, refit = sizes[it]
            it += 1
            given = picks[pos: pos + kk]
            cs = np.where(selected, -np.inf, sc)
            order = np.lexsort((np.arange(T), -cs))
            top = float(cs[order[0]])
            if set(given) != set(int(j) for j in order[:kk]):
                out = ~selected
                out[given] = False
                c_out, b_out = cs[out], b_all[out]
                thr = MARGIN_TOL * abs(top)
                resolved = any(np.any((c_out - cs[g] > thr) & (c_out - cs[g] > eb * (b_out + b_all[g])))
                               for g in given)
                (rep["mismatch_iters"] if resolved else rep["forced_iters"]).append(it)
            selected[given] = True
            pos += kk
            if refit:
                break
        rep["cycles"][c] = cyc
    rep["weights_ok"], rep["relres_ok"] = True, True
    rep["e_mass_diff"] = rep["e_out_diff"] = 0.0
    if final:
        Ck, beta, Cv, sel = head_outputs(res, h)
        rep["same_set"] = bool(np.array_equal(np.sort(np.asarray(picks)), sel))
        P = Phi[:, sel]
        w_ref = O.nnls_exact(P, m)
        beta_ref = O.log_weights(w_ref)
        if beta_in is not None:
            beta_ref = beta_ref + np.asarray(beta_in, dtype=np.float64)[sel]
        ref_out = (np.asarray(K, dtype=np.float64)[sel], beta_ref, O.ols_values(P, w_ref, feats.Y))
        order = np.argsort(np.asarray(picks), kind="stable")
        w_gpu64 = np.asarray(trace["weight"][h], dtype=np.float64)[order]
        relres_gpu = float(relres_tr[-1]) if len(relres_tr) else None
        _judge_weights(rep, Q, K, V, P, m, feats.Y, w_ref, ref_out, sel, Ck, beta, Cv, w_gpu64, relres_gpu, beta_in)
        rep["ck_exact"] = bool(np.array_equal(Ck, ref_out[0]))
        REPORTS.append(rep)
    rep["ok"] = (not rep["mismatch_iters"] and rep["weights_ok"] and rep["relres_ok"] and
                 rep["e_mass_diff"] <= ERR_TOL and rep["e_out_diff"] <= ERR_TOL and
                 rep.get("same_set", True) and rep.get("ck_exact", True))
    return rep


def _judge_weights(rep, Q, K, V, P, m, Y, w_ref, ref_out, sel, Ck, beta, Cv, w_gpu64, relres_gpu, beta_in):
    """The weight and error part of the replay (see the module docstring) for
    the GPU's key set `sel` (ascending), its outputs (Ck, beta, Cv), its
    float64 weights w_gpu64 (ascending key order) and the relative residual
    its trace reports after the last refit, against the oracle's exact
    minimiser w_ref on the same keys (P = Phi[:, sel]) and the oracle's
    outputs ref_out = (Ck, beta, Cv).  Fills rep; rep['weights_ok'] is the
    weight verdict."""
    # weights: the GPU's beta carries beta_in + log w
    bi = np.zeros(len(sel)) if beta_in is None else np.asarray(beta_in, dtype=np.float64)[sel]
    with np.errstate(invalid="ignore"):
        w_gpu = np.where(np.isfinite(beta), np.exp(beta - bi), 0.0)
    act_g, act_r = w_gpu > 0, w_ref > 0
    both = act_g & act_r
    ref_beta = ref_out[1]
    rep["beta_maxdiff"] = float(np.max(np.abs(beta[both] - ref_beta[both]))) if np.any(both) else 0.0
    rep["one_sided_ok"] = _one_sided_ok(w_gpu, w_ref)
    res_g = float(np.linalg.norm(m - P @ w_gpu64))
    res_r = float(np.linalg.norm(m - P @ w_ref))
    rep["resid_excess"] = (res_g - res_r) / max(res_r, 1e-300)
    rep["rel_resid"] = res_r / float(np.linalg.norm(m))
    # the trace's relative residual after the last refit is that of the GPU's
    # own weights (float64 residuals on both sides; cancellation leaves about
    # 1e-16 / relres of relative difference)
    rep["relres_ok"] = True
    if relres_gpu is not None:
        want = res_g / float(np.linalg.norm(m))
        rep["relres_gpu"] = relres_gpu
        rep["relres_ok"] = abs(relres_gpu - want) <= 1e-6 * want + 1e-13
    e_gpu = oracle.errors(Q, K, V, Ck, beta, Cv, beta_in)
    e_ref = oracle.errors(Q, K, V, ref_out[0], ref_beta, ref_out[2], beta_in)
    rep["e_gpu"], rep["e_ref"] = e_gpu, e_ref
    rep["e_mass_diff"] = abs(e_gpu[0] - e_ref[0])
    rep["e_out_diff"] = abs(e_gpu[1] - e_ref[1])
    rep["fallback"] = False
    rep["beta_envelope"] = None
    rep["reference"] = ref_out  # the compaction the GPU's errors are compared with
    weights_ok = rep["beta_maxdiff"] <= BETA_TOL and rep["one_sided_ok"]
    if not weights_ok:
        # Is beta determined by the float64 data?  Not when the columns of
        # both supports together are numerically dependent (their smallest
        # singular value, unit columns, below NULL_SV: the NNLS minimisers form
        # a face and the two weight vectors are both on it), nor when the same
        # NNLS solved again in extended precision moves beta past the tolerance.
        U = (w_gpu64 > 0) | (w_ref > 0)
        Pu = P[:, U]
        nrm = np.linalg.norm(Pu, axis=0)
        sv = np.linalg.svd(Pu / np.where(nrm > 0, nrm, 1.0), compute_uv=False) if Pu.shape[1] else np.ones(1)
        # more columns than queries: dependent whatever the singular values say
        rep["union_sv_min"] = float(sv[-1] / sv[0]) if Pu.shape[1] <= Pu.shape[0] else 0.0
        if len(w_ref) <= LD_MAX_T:
            w_ld = O.nnls_qr(P, m, w0=w_ref, dtype=np.longdouble)
        else:
            # past the size an extended-precision solve affords: the same
            # NNLS on data moved by its float64 rounding (each entry of Phi_S
            # and m by a relative 2^-52, seeded), warm-started at the minimiser
            rng = np.random.default_rng(len(w_ref))
            eps = np.finfo(np.float64).eps
            w_ld = O.nnls_exact(P * (1 + eps * rng.uniform(-1, 1, P.shape)), m * (1 + eps * rng.uniform(-1, 1, m.shape)),
                                w_prev=w_ref)
        both_o = (w_ref > 0) & (w_ld > 0)
        env = float(np.max(np.abs(np.log(w_ref[both_o]) - np.log(w_ld[both_o])))) if np.any(both_o) else 0.0
        if not _one_sided_ok(w_ld, w_ref):
            env = float("inf")
        rep["beta_envelope"] = env
        if rep["union_sv_min"] < NULL_SV or (env is not None and env > BETA_TOL):
            rep["fallback"] = True
            weights_ok = rep["resid_excess"] <= RESID_REL
            # the minimisers form a face and the value fit depends on which
            # point of it the weights are: the oracle's own value fit, taken on
            # the GPU's weights, is the reference for the GPU's errors
            Cv_face = O.ols_values(P, w_gpu64, Y)
            e_face = oracle.errors(Q, K, V, Ck, beta, Cv_face, beta_in)
            rep["e_face"] = e_face
            rep["reference"] = (Ck, beta, Cv_face)
            rep["e_mass_diff"] = abs(e_gpu[0] - e_face[0])
            rep["e_out_diff"] = abs(e_gpu[1] - e_face[1])
    rep["weights_ok"] = bool(weights_ok)


def _one_sided_ok(wa, wb):
    """A key active on one side only carries at most WEIGHT_REL of that side's largest weight."""
    only_a = (wa > 0) & ~(wb > 0)
    only_b = (wb > 0) & ~(wa > 0)
    return bool(np.all(wa[only_a] <= WEIGHT_REL * wa.max(initial=0.0)) and
                np.all(wb[only_b] <= WEIGHT_REL * wb.max(initial=0.0)))


def assert_fallback_share(reports, share=FALLBACK_SHARE):
    """At most ``share`` of a test's heads may be held to the NNLS minimum
    value instead of the beta rule."""
    n_fb = sum(1 for r in reports if r.get("fallback"))
    assert n_fb <= share * len(reports), f"{n_fb} of {len(reports)} heads needed the residual gate"
