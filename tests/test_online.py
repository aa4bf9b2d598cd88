"""The online re-compaction loop: its schedule (CPU) and each round on the
GPU against the oracle, with the bias of earlier rounds carried as beta_in."""
import os

import numpy as np
import pytest
import torch

import synth
from attention_matching_least_amd import amc, online
from oracle import amc_oracle as O

from amc_check import replay_check, to_device

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_schedule.txt")


def _golden():
    g = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            g[k] = float(v)
    return g


def test_schedule_matches_oracle_and_pages():
    g = _golden()
    phys, keep, rounds = int(g["physical"]), int(g["keep_newest"]), int(g["rounds"])
    got = online.represented_tokens(phys, keep, rounds, g["ratio"])
    assert got == O.online_effective_length(phys, keep, rounds, g["ratio"])
    # the pages round the effective length to 8192; the schedule gives 8132
    assert abs(got - g["effective_reported"]) / g["effective_reported"] < 0.01
    assert online.round_budget(4076, 0.5) == 2038


def _host(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


@pytest.mark.gpu
def test_online_rounds_match_oracle():
    """Two rounds over two heads: a 1024-token cache, keep 20, each round
    compacts 1004 keys to 502 (the pages' 50%) with 2048 fresh queries.
    Every round's inputs (the GPU's own cache, with the bias of the round
    before) are replayed through the oracle.  At this size a 50% budget fits
    the mass almost exactly, so the heads' refits leave the Gram form for
    the orthogonal-factorisation path."""
    w = synth.online_workload(num_heads=2, L=1024, n=2048, d=128, rounds=2, seed_root=61)
    heads = w.initial()
    H, L, d = w.num_heads, w.L, w.d
    budget = online.round_budget(L - w.keep_newest, w.ratio)
    nfree = L - budget - w.keep_newest
    toks = {(r, h): w.round_tokens(r, h, heads[h].centres, nfree) for r in range(w.rounds) for h in range(H)}
    cache = online.Cache(torch.stack([to_device(h.K, "bf16") for h in heads]),
                         torch.stack([to_device(h.V, "bf16") for h in heads]),
                         torch.zeros((H, L), dtype=torch.float32, device="cuda"))

    def queries(r):
        return torch.stack([to_device(toks[r, h][0], "bf16") for h in range(H)])

    def fresh(r, count):
        assert count == nfree
        return (torch.stack([to_device(toks[r, h][1], "bf16") for h in range(H)]),
                torch.stack([to_device(toks[r, h][2], "bf16") for h in range(H)]))

    print(f"online loop: H={H} L={L} budget={budget} rounds={w.rounds}", flush=True)
    out = online.online_loop(cache, queries, fresh, w.rounds, keep_newest=w.keep_newest, ratio=w.ratio,
                             topk=w.topk, refit_every=w.refit_every, keep_inputs=True, trace=True)
    torch.cuda.synchronize()
    dead = 0
    for r, rd in enumerate(out.rounds):
        Q, Kp, Vp, bp = rd.inputs
        hs = rd.result.head_status.cpu().numpy()
        assert np.all(hs & ~(amc.HS_CHOL_JITTER | amc.HS_NNLS_SINGULAR | amc.HS_NNLS_QR) == 0), hs
        tr = rd.result.trace()
        if r > 0:
            assert np.any(_host(bp) != 0.0)  # the bias of the earlier round is carried
        for h in range(H):
            bi = _host(bp[h])
            dead += int(np.sum(np.isneginf(bi)))
            rep = replay_check(_host(Q[h]), _host(Kp[h]), _host(Vp[h]), budget, w.topk, w.refit_every, rd.result,
                               h, beta_in=bi, trace=tr)
            print(f"round {r} head {h}: {rep}", flush=True)
            assert rep["ok"], (r, h, rep)
    print(f"dead keys carried into later rounds: {dead}", flush=True)
    # the final cache: last round's compacted block, then the newest tokens, then the refill
    last = out.rounds[-1].result
    fin = out.cache
    assert fin.length == L
    assert torch.equal(fin.K[:, :budget].reshape(-1, d), last.Ck)
    assert torch.equal(fin.beta[:, :budget].reshape(-1), last.beta)
    assert torch.all(fin.beta[:, budget + w.keep_newest:] == 0)
