"""Seeded synthetic inputs for attention-matching KV compaction.

This module holds no arithmetic of the compaction method: it only draws
random numbers, rounds them to the storage format and lays them out.  Both
the float64 oracle (``oracle/``) and the HIP path's tests and benchmark take
their inputs from here, so the two sides see bit-identical values.

Recipe, per KV head (one ``numpy.random.default_rng`` per head, draws in
this order):

1. cluster centres ``C ~ N(0, 1.5^2)``, shape (8, d);
2. key cluster ids ``u_k ~ U{0..7}``, length T;
3. keys ``K = C[u_k] + N(0, 0.5^2)``, shape (T, d);
4. with outliers: key channels 0 and 1 are multiplied by 8;
5. query cluster ids ``u_q ~ U{0..7}``, length n;
6. queries ``Q = N(0, 1) + C[u_q]``, shape (n, d);
7. values ``V ~ N(0, 1)``, shape (T, d).

Values are cast float64 -> float32 -> bfloat16 with round-to-nearest-even
for the bf16 workloads, or float64 -> float32 for the fp32 one.  Every
array is returned as float64 holding exactly the stored values.

The shapes stand in for the pages' workloads (Qwen3-4B-shaped GQA heads:
d=128, 8 KV heads per layer, 36 layers; QuALITY-length contexts at T=8192,
LongHealth-length at T=60000).  Real activations need trained weights that
are not available, so clustered Gaussians take their place.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

N_CLUSTERS = 8


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def f32_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest float32 -> float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE); returns the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 (via float32, both round-to-nearest-even) -> float64."""
    return bf16_to_f64(bf16_bits(x))


def store_round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return f32_round(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------
# one head
# ----------------------------------------------------------------------------
@dataclass
class Head:
    Q: np.ndarray  # (n, d) float64 holding stored values
    K: np.ndarray  # (T, d)
    V: np.ndarray  # (T, d)
    centres: np.ndarray  # (8, d) float64, unrounded (used to draw fresh tokens)
    outliers: bool = False


def _draw_head(rng: np.random.Generator, n: int, T: int, d: int, outliers: bool):
    C = rng.normal(0.0, 1.5, size=(N_CLUSTERS, d))
    uk = rng.integers(0, N_CLUSTERS, size=T)
    K = C[uk] + rng.normal(0.0, 0.5, size=(T, d))
    if outliers:
        K[:, 0:2] *= 8.0
    uq = rng.integers(0, N_CLUSTERS, size=n)
    Q = rng.normal(0.0, 1.0, size=(n, d)) + C[uq]
    V = rng.normal(0.0, 1.0, size=(T, d))
    return Q, K, V, C


def make_head(seed, n: int, T: int, d: int, outliers: bool, dtype: str) -> Head:
    """One head from ``seed`` (an int, a list of ints or a SeedSequence)."""
    rng = np.random.default_rng(seed)
    Q, K, V, C = _draw_head(rng, n, T, d, outliers)
    return Head(store_round(Q, dtype), store_round(K, dtype), store_round(V, dtype), C, outliers)


def fresh_tokens(seed, centres: np.ndarray, n_q: int, n_kv: int, outliers: bool, dtype: str):
    """Fresh queries and key/value tokens that reuse a head's cluster centres.

    Draw order: key cluster ids, keys, query cluster ids, queries, values.
    """
    rng = np.random.default_rng(seed)
    d = centres.shape[1]
    uk = rng.integers(0, N_CLUSTERS, size=n_kv)
    K = centres[uk] + rng.normal(0.0, 0.5, size=(n_kv, d))
    if outliers:
        K[:, 0:2] *= 8.0
    uq = rng.integers(0, N_CLUSTERS, size=n_q)
    Q = rng.normal(0.0, 1.0, size=(n_q, d)) + centres[uq]
    V = rng.normal(0.0, 1.0, size=(n_kv, d))
    return store_round(Q, dtype), store_round(K, dtype), store_round(V, dtype)


def digit_variant_head(seed, n: int, T: int, d: int, kind: str) -> Head:
    """A bf16 head whose rows exercise the exact-digit logit kernel's cases.

    kind "z2": every entry within a factor 2 of its row's largest (its two low
    base-256 digits are zero); "z1" / "z0": magnitudes log-uniform over 2^-15
    / 2^-24 of the largest (one / no low digit zero); "offgrid": as "z1" with
    one query entry 2^-40 below its row's largest (off the 38-bit digit grid,
    so the head takes the float64 logit kernel).  Values are plain random
    draws, bf16-rounded.
    """
    rng = np.random.default_rng(seed)
    span = {"z2": 1.0, "z1": 15.0, "z0": 24.0, "offgrid": 15.0}[kind]

    def rows(m):
        mag = np.exp2(-rng.uniform(0.0, span, size=(m, d)))
        mag[:, 0] = 1.0  # each row's largest
        x = rng.choice([-1.0, 1.0], size=(m, d)) * mag * 1.5
        return x

    Q, K, V = rows(n), rows(T) * 0.25, rng.normal(0.0, 1.0, size=(T, d))
    if kind == "offgrid":
        Q[n // 2, 3] = 1.5 * 2.0 ** -40
    Qb, Kb, Vb = store_round(Q, "bf16"), store_round(K, "bf16"), store_round(V, "bf16")
    return Head(Qb, Kb, Vb, np.zeros((1, d)), False)


def sensitivity_curves(seed, num_heads: int, steps: int) -> np.ndarray:
    """Synthetic per-head sensitivity curves for the budget schedule (real ones
    need a model): loss_h(j) = a_h exp(-(j+1) / s_h), j = 0..steps-1, a
    decreasing convex curve per head with a log-normal level a_h and a decay
    length s_h uniform in [1, steps / 2]: some heads need many keys, others few."""
    rng = np.random.default_rng(seed)
    a = np.exp(rng.normal(0.0, 1.0, size=num_heads))
    sc = rng.uniform(1.0, max(1.0, steps / 2), size=num_heads)
    j = np.arange(1, steps + 1)
    return a[:, None] * np.exp(-j[None, :] / sc[:, None])


def random_beta(seed, T: int, scale: float = 1.0) -> np.ndarray:
    """A float32-representable per-key bias, for re-compaction inputs."""
    rng = np.random.default_rng(seed)
    return f32_round(rng.normal(0.0, scale, size=T))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    num_heads: int
    n: int
    T: int
    d: int
    budgets: List[int]
    topk: int
    refit_every: int
    dtype: str
    outliers: bool
    seed_root: int
    description: str = ""
    recompute: bool = False
    extra: dict = field(default_factory=dict)

    def head_seeds(self):
        if self.num_heads == 1 and self.seed_root == 0:
            return [np.random.SeedSequence(0)]
        return np.random.SeedSequence(self.seed_root).spawn(self.num_heads)

    def head(self, h: int) -> Head:
        return make_head(self.head_seeds()[h], self.n, self.T, self.d, self.outliers, self.dtype)

    def heads(self, which: Optional[List[int]] = None) -> List[Head]:
        seeds = self.head_seeds()
        idx = range(self.num_heads) if which is None else which
        return [make_head(seeds[h], self.n, self.T, self.d, self.outliers, self.dtype) for h in idx]


def dirichlet_budgets(num_heads: int, T: int, ratio: int = 20, lo: int = 8, hi: int = 2048,
                      seed=(4, 1)) -> List[int]:
    """Per-head budgets: a Dirichlet(0.5) split of num_heads*T/ratio keys,
    rounded half-to-even and clamped to [lo, hi] with no redistribution."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    p = rng.dirichlet([0.5] * num_heads)
    total = num_heads * T / ratio
    b = np.clip(np.round(p * total), lo, hi).astype(np.int64)
    return [int(x) for x in b]


def workload(idx: int) -> Workload:
    """The five seeded workloads (0: tiny fp32 head; 1: one layer; 2: a full
    36x8-head stack with batched selection; 3: 60k-token stack; 4: varlen
    Dirichlet budgets)."""
    if idx == 0:
        return Workload("single-head-fp32-T512", 1, 256, 512, 64, [32], 1, 1, "f32", False, 0,
                        "1 head, d=64, T=512, n=256, t=32 (16x), plain OMP, fp32")
    if idx == 1:
        return Workload("qwen3-4b-layer-T8192-50x", 8, 4096, 8192, 128, [164] * 8, 1, 1, "bf16", True, 1,
                        "8 KV heads, d=128, T=8192, n=4096, t=164 (50x), plain OMP, bf16")
    if idx == 2:
        return Workload("qwen3-4b-stack-T8192-50x", 288, 4096, 8192, 128, [164] * 288, 4, 2, "bf16", True, 2,
                        "288 KV heads (36 layers x 8), d=128, T=8192, n=4096, t=164 (50x), "
                        "batched selection top-k=4, refit every 2 iterations, bf16")
    if idx == 3:
        return Workload("qwen3-4b-stack-T60000-10x", 288, 8192, 60000, 128, [6000] * 288, 32, 4, "bf16", True, 3,
                        "288 KV heads, d=128, T=60000, n=8192, t=6000 (10x), top-k=32, refit every 4, "
                        "Phi recomputed", recompute=True)
    if idx == 4:
        return Workload("qwen3-4b-stack-T8192-varlen", 288, 4096, 8192, 128, dirichlet_budgets(288, 8192),
                        4, 2, "bf16", True, 4,
                        "288 KV heads, d=128, T=8192, n=4096, Dirichlet(0.5) budgets in [8, 2048]")
    raise ValueError(idx)


def scaled_workload(idx: int, num_heads: int, n: int, T: int, budget: int, d: Optional[int] = None) -> Workload:
    """Same recipe and selection settings as ``workload(idx)`` at a smaller shape (for tests)."""
    w = workload(idx)
    return Workload(w.name + f"-scaled-H{num_heads}-n{n}-T{T}-t{budget}", num_heads, n, T,
                    w.d if d is None else d, [budget] * num_heads, w.topk, w.refit_every, w.dtype,
                    w.outliers, 100 + idx, w.description + " (scaled)")


# ----------------------------------------------------------------------------
# online re-compaction loop (the varlen stack's second workload)
# ----------------------------------------------------------------------------
@dataclass
class OnlineWorkload:
    """A fixed physical cache of L tokens per head, re-compacted `rounds`
    times: each round compacts all but the newest `keep_newest` tokens by
    `ratio` with n fresh reference queries, then fresh tokens refill it."""
    name: str
    num_heads: int
    L: int
    n: int
    d: int
    rounds: int
    keep_newest: int
    ratio: float
    topk: int
    refit_every: int
    seed_root: int
    dtype: str = "bf16"

    def head_seeds(self):
        return np.random.SeedSequence(self.seed_root).spawn(self.num_heads)

    def initial(self, which: Optional[List[int]] = None) -> List[Head]:
        """The starting caches: T = L tokens of each head (its queries are unused)."""
        seeds = self.head_seeds()
        idx = range(self.num_heads) if which is None else which
        return [make_head(seeds[h], self.n, self.L, self.d, True, self.dtype) for h in idx]

    def round_tokens(self, r: int, h: int, centres: np.ndarray, n_fresh: int):
        """(Q, K_new, V_new) of round r for head h: the reference queries of
        the round and the tokens decoded after it."""
        return fresh_tokens(np.random.SeedSequence([self.seed_root, 2, r, h]), centres, self.n, n_fresh, True,
                            self.dtype)


def online_workload(num_heads: int = 288, L: int = 4096, n: int = 4096, d: int = 128, rounds: int = 6,
                    seed_root: int = 4) -> OnlineWorkload:
    """Default: 288 heads, a 4096-token cache, 6 rounds of 50% keeping the
    newest 20 (so T = 4076 -> t = 2038 per round), n = 4096, top-k 4, refit
    every 2 iterations, bf16."""
    return OnlineWorkload(f"qwen3-4b-stack-online-L{L}-x{rounds}", num_heads, L, n, d, rounds, 20, 0.5, 4, 2,
                          seed_root)
