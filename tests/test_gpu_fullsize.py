"""Full-size heads whose budgets pass the orthogonal-factorisation refit's
limit (640 keys), replayed against the oracle at chosen refits
(amc_check.spot_replay): a 2048-key head of the varlen stack, one round of
the online loop at its full size (4076 keys to 2038), and two heads of the
60k-token stack (a recorded limit of the Gram-form refit)."""
import numpy as np
import pytest
import torch

import synth
from attention_matching_least_amd import amc, online

from amc_check import pack_heads, spot_replay

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(msg):
    print(msg, flush=True)


def _compact(heads, budgets, k, R, beta_in=None, **kw):
    Q, K, V, cu_q, cu_k = pack_heads(heads, "bf16")
    res = amc.compact(Q, K, V, budgets, cu_q=cu_q, cu_k=cu_k, beta_in=beta_in, select="batched", topk=k,
                      refit_every=R, trace=True, **kw)
    torch.cuda.synchronize()
    hs = res.head_status.cpu().numpy()
    assert np.all(hs & (amc.HS_NNLS_CAP | amc.HS_NONFINITE) == 0), hs
    return res


def _report(tag, rep):
    cyc = {c: {k: (round(v, 9) if isinstance(v, float) else v) for k, v in d.items()} for c, d in rep["cycles"].items()}
    keys = ("ok", "mismatch_iters", "forced_iters", "beta_maxdiff", "one_sided_ok", "fallback", "union_sv_min",
            "resid_excess", "rel_resid", "relres_gpu", "e_mass_diff", "e_out_diff", "same_set")
    _say(f"{tag}: cycles {cyc}; " + ", ".join(f"{k} {rep.get(k)}" for k in keys))


def test_varlen_2048_key_head():
    """The first 2048-key head of the varlen stack (T=8192, n=4096, top-k 4,
    refit every 2: 256 refits), at refits 1, 64, 128 and 192 and after the
    last.  Its refits are the Gram form's; the polish refit's entering test
    resolves any gradient the float64 data do (with the selection refits'
    test, 10 eps t, it ended with beta off by 0.11 at a residual 1.6e-8 above
    the minimum)."""
    w = synth.workload(4)
    h = w.budgets.index(2048)
    head = w.head(h)
    _say(f"varlen head {h}: t=2048 T={w.T} n={w.n}")
    res = _compact([head], [2048], w.topk, w.refit_every)
    rep = spot_replay(head.Q, head.K, head.V, 2048, w.topk, w.refit_every, res, 0, [1, 64, 128, 192])
    _report(f"varlen head {h}", rep)
    assert rep["ok"], rep


def test_online_round_full_size():
    """The first round of the online loop at its full size for one head: the
    4076 oldest tokens of a 4096-token cache (the newest 20 kept) compacted
    to 2038 with 4096 fresh reference queries, top-k 4, refit every 2 (255
    refits), at refits 1, 64, 128 and 192 and after the last.  The loop's
    first round is exactly this compaction (no bias carried yet)."""
    w = synth.online_workload()
    head = w.initial([0])[0]
    T = w.L - w.keep_newest
    t = online.round_budget(T, w.ratio)
    nfree = w.L - t - w.keep_newest
    Qr = w.round_tokens(0, 0, head.centres, nfree)[0]
    inp = synth.Head(Qr, head.K[:T], head.V[:T], head.centres, True)
    _say(f"online round 1: T={T} -> t={t}, n={Qr.shape[0]}")
    res = _compact([inp], [t], w.topk, w.refit_every)
    rep = spot_replay(inp.Q, inp.K, inp.V, t, w.topk, w.refit_every, res, 0, [1, 64, 128, 192])
    _report("online round 1", rep)
    assert rep["ok"], rep


@pytest.fixture(scope="module")
def long_context_run():
    """Two heads of the 60k-token stack compacted in one call."""
    w = synth.workload(3)
    heads = w.heads([0, 1])
    _say(f"60k-token heads 0, 1: t={w.budgets[0]}, {w.budgets[1]}")
    return w, heads, _compact(heads, w.budgets[:2], w.topk, w.refit_every)


@pytest.mark.xfail(strict=True, reason="past 640 keys the refit takes the Gram form, which in this regime (relative "
                   "residual near 6e-7) stops above the NNLS minimum (16% at refit 12), so later picks differ")
@pytest.mark.parametrize("h", [0, 1])
def test_long_context_head(long_context_run, h):
    """A head of the 60k-token stack (T=60000, n=8192, t=6000, top-k 32,
    refit every 4: 47 refits), at refits 1 and 12.  A recorded limit:
    the refits are the Gram form's."""
    w, heads, res = long_context_run
    head = heads[h]
    rep = spot_replay(head.Q, head.K, head.V, w.budgets[h], w.topk, w.refit_every, res, h, [1, 12],
                      final=False)
    _report(f"60k-token head {h}", rep)
    assert rep["ok"], rep


def test_long_context_head_fine_entering_test():
    """The first head of the 60k-token stack with the Gram solver's entering
    test given as 1e-14 of max |b| in every refit (amc_options.nnls_tol; at
    most 400 active-set steps per refit) instead of the default 10 eps t: its
    picks follow the oracle's at refits 12 and 24, where the default's part
    from the oracle's after refit 12.  The finer test costs about four times
    the default's time per head."""
    w = synth.workload(3)
    head = w.heads([0])[0]
    _say(f"60k-token head 0, entering test 1e-14: t={w.budgets[0]}")
    res = _compact([head], w.budgets[:1], w.topk, w.refit_every, nnls_tol=1e-14, nnls_max_iters=400)
    rep = spot_replay(head.Q, head.K, head.V, w.budgets[0], w.topk, w.refit_every, res, 0, [12, 24], final=False)
    _report("60k-token head 0, entering test 1e-14", rep)
    assert rep["ok"], rep
