"""Online re-compaction of a fixed-size KV cache during decoding
(zhichai.net deep-dive, section 2.4, the AIME online experiment; xinfinite.net
article, section 5 and Table 3: whenever the physical cache is full,
everything but the newest 20 tokens is compacted by 50% and decoding refills
the freed slots, up to six times).

Each round runs one libamc compaction over every head's prefix, carrying the
prefix's per-key bias (beta) from the earlier rounds as beta_in, so that a key
that already stands for several originals keeps its weight.  The compacted
keys, their new bias and their fitted values replace the prefix; the newest
tokens stay as they were; fresh tokens fill the cache back to its physical
length.  Everything stays in device memory; this module only slices and
concatenates buffers and calls the library, which does all of the arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Tuple

import torch

from . import amc


@dataclass
class Cache:
    """A batch of per-head caches of one physical length L."""
    K: torch.Tensor      # [H][L][d] storage dtype
    V: torch.Tensor      # [H][L][d] storage dtype
    beta: torch.Tensor   # [H][L] float32 (0 for plain tokens, -inf for dead keys)

    @property
    def length(self) -> int:
        return int(self.K.shape[1])


@dataclass
class Round:
    budget: int
    prefix: int
    result: amc.CompactResult
    inputs: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]] = None


@dataclass
class LoopResult:
    cache: Cache
    rounds: List[Round] = field(default_factory=list)


def round_budget(prefix: int, ratio: float) -> int:
    """Keys kept from a prefix of the given length (at least one)."""
    return max(1, int(round(prefix * ratio)))


def online_loop(cache: Cache, queries: Callable[[int], torch.Tensor],
                fresh: Callable[[int, int], Tuple[torch.Tensor, torch.Tensor]], rounds: int, *,
                keep_newest: int = 20, ratio: float = 0.5, topk: int = 4, refit_every: int = 2,
                keep_inputs: bool = False, trace: bool = False, timer: Optional[amc.Timer] = None,
                workspace: Optional[torch.Tensor] = None) -> LoopResult:
    """Runs ``rounds`` online compactions of ``cache``.

    queries(r) -> [H][n][d] reference queries for round r (storage dtype).
    fresh(r, count) -> (K, V), each [H][count][d]: the tokens decoded after
    round r, appended with beta = 0.
    keep_inputs: keep each round's (Q, K prefix, V prefix, beta prefix), for
    checking a round on its own.
    """
    H, L, d = (int(x) for x in cache.K.shape)
    if cache.V.shape != cache.K.shape or tuple(cache.beta.shape) != (H, L):
        raise ValueError("cache K, V, beta shapes disagree")
    if not 0 <= keep_newest < L:
        raise ValueError("keep_newest must leave a non-empty prefix")
    if not 0.0 < ratio < 1.0:
        raise ValueError("ratio must lie in (0, 1)")
    select = "omp" if (topk == 1 and refit_every == 1) else "batched"
    prefix = L - keep_newest
    budget = round_budget(prefix, ratio)
    out = LoopResult(cache)
    if workspace is None and rounds > 0:
        # one workspace serves every round (the problem shape does not change)
        n = int(queries(0).shape[1])
        nb = amc.compact_workspace_bytes([n * h for h in range(H + 1)], [prefix * h for h in range(H + 1)],
                                         [budget] * H, d, cache.K.dtype, select=select, topk=topk,
                                         refit_every=refit_every, cv_dtype=cache.K.dtype)
        workspace = torch.empty(nb + 256, dtype=torch.uint8, device=cache.K.device)
    for r in range(rounds):
        Q = queries(r)
        if Q.dim() != 3 or Q.shape[0] != H or Q.shape[2] != d or Q.dtype != cache.K.dtype:
            raise ValueError("queries(r) must be [H][n][d] in the cache's dtype")
        Kp = cache.K[:, :prefix].contiguous()
        Vp = cache.V[:, :prefix].contiguous()
        bp = cache.beta[:, :prefix].contiguous()
        res = amc.compact(Q, Kp, Vp, budget, beta_in=bp.reshape(-1), select=select, topk=topk,
                          refit_every=refit_every, cv_dtype=cache.K.dtype, trace=trace, timer=timer,
                          workspace=workspace)
        kept = (Q, Kp, Vp, bp) if keep_inputs else None
        out.rounds.append(Round(budget, prefix, res, kept))
        nfree = L - budget - keep_newest
        Kn, Vn = fresh(r, nfree)
        if Kn.shape != (H, nfree, d) or Vn.shape != (H, nfree, d):
            raise ValueError("fresh(r, count) must return two [H][count][d] tensors")
        cache = Cache(
            torch.cat([res.Ck.view(H, budget, d), cache.K[:, prefix:], Kn.to(cache.K.dtype)], dim=1),
            torch.cat([res.Cv.view(H, budget, d), cache.V[:, prefix:], Vn.to(cache.V.dtype)], dim=1),
            torch.cat([res.beta.view(H, budget), cache.beta[:, prefix:],
                       torch.zeros((H, nfree), dtype=torch.float32, device=cache.beta.device)], dim=1))
        out.cache = cache
    return out


def represented_tokens(physical: int, keep_newest: int, rounds: int, ratio: float = 0.5) -> int:
    """Tokens the cache stands for after ``rounds`` compactions: the physical
    length plus the slots each round frees."""
    prefix = physical - keep_newest
    return physical + rounds * (prefix - round_budget(prefix, ratio))
