"""Throughput benchmark of attention-matching KV compaction on one MI355X.

A step is one amc_compact call over the whole batch of heads (every stage:
shift, mass features, the selection loop with its NNLS refits, the value fit
and the packing), with inputs already resident in HBM.  The default workload
is a Qwen3-4B-shaped stack: 36 layers x 8 KV heads = 288 heads, T = 8192 keys,
n = 4096 reference queries, d = 128, budget 164 (50x), batched selection with
top-k = 4 and a refit every 2 iterations, bf16 inputs.

Prints one JSON line (rank 0).  The timed steps run as the library runs by
default (large stacks in four head groups on separate streams, whose kernels
overlap).  A kernel pass then times the same steps again with the heads in one
group and the library's HIP-event timer attached, so that every event pair
brackets one kernel running alone: the per-kernel times and the dominant
kernel's roofline figure come from it.  The CPU baseline is the float64 oracle
on a small seeded sample of the same heads.

The same run (default workload, unless --no-long) also measures the metric's
second half: the wall-clock seconds of compacting the 60k-token stack (288
heads, T = 60000, n = 8192, t = 6000, top-k 32, refit every 4, Phi recomputed
in every sweep), reported under "long_context".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
F64_MFMA_PEAK_TFS = 78.6
I8_MFMA_PEAK_TOPS = 5000.0  # dense int8 matrix peak of the MI355X
BF16_MFMA_PEAK_TFS = 2500.0  # dense bf16 matrix peak of the MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_qwen3-4b-stack-T8192-50x.md")
KERNEL_SOURCES = {"k_sweep": os.path.join(ROOT, "attention_matching_least_amd", "csrc", "k_select.hip"),
                  "k_phi": os.path.join(ROOT, "attention_matching_least_amd", "csrc", "k_phi.hip")}


def _head_bits(args):
    idx, h = args
    w = synth.workload(idx)
    head = w.head(h)
    return (synth.bf16_bits(head.Q), synth.bf16_bits(head.K), synth.bf16_bits(head.V)) if w.dtype == "bf16" else \
        (head.Q.astype(np.float32), head.K.astype(np.float32), head.V.astype(np.float32))


def generate(idx: int, workers: int):
    w = synth.workload(idx)
    H = w.num_heads
    jobs = [(idx, h) for h in range(H)]
    if workers > 1 and H > 1:
        with ProcessPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(_head_bits, jobs, chunksize=max(1, H // (4 * workers))))
    else:
        parts = [_head_bits(j) for j in jobs]
    Q = np.concatenate([p[0] for p in parts])
    K = np.concatenate([p[1] for p in parts])
    V = np.concatenate([p[2] for p in parts])
    return w, Q, K, V


# 2^(bit length - 1) of a 1..255 significand
_TOPBIT = np.array([0] + [int(v).bit_length() - 1 for v in range(1, 256)], dtype=np.int32)


def digit_zeros(bits: np.ndarray):
    """Per row of bf16 bit patterns, as the int8 logit kernel sees it: z = the
    low base-256 digits that are zero in all entries of the row (up to 2;
    rows on the digit grid of 2^(E - 37), E the row's largest exponent), and
    whether the row is off that grid (or non-finite)."""
    zs, bads = [], []
    for r0 in range(0, bits.shape[0], 32768):
        b = bits[r0:r0 + 32768].astype(np.int32)
        ef, mt = (b >> 7) & 0xff, b & 0x7f
        nz = (b & 0x7fff) != 0
        p = np.where(ef == 0, -133, ef - 134)
        e = p + _TOPBIT[np.where(ef == 0, mt, mt | 0x80)]
        E = np.where(nz, e, -100000).max(axis=1)
        pmin = np.where(nz, p, 100000).min(axis=1)
        anynz = nz.any(axis=1)
        E = np.where(anynz, E, 0)
        z = np.where(anynz, np.clip((pmin + 37 - E) >> 3, 0, 2), 2)
        bad = (anynz & (pmin < E - 37)) | (ef == 255).any(axis=1)
        zs.append(z)
        bads.append(bad)
    return np.concatenate(zs), np.concatenate(bads)


def phi_matrix_ops(Qb: np.ndarray, Kb: np.ndarray, w) -> float:
    """Matrix-core work of one mass-feature pass over the stack, in int8-equivalent
    operations: per head on the digit grid, for every wave of 16 queries and
    16-key block, (d / 64) (5 - zq) (5 - zk) int8 16x16x64 products (zq, zk the
    wave's and the block's all-zero low digits), and 6 d / 16 bf16 16x16x32
    products of the Phi V split per wave and 64-key tile (a bf16 operation
    counting as two at half the int8 rate).  Heads off the grid (float64
    kernel) are left out."""
    H, n, T, d = w.num_heads, w.n, w.T, w.d
    zq, bq = digit_zeros(Qb)
    zk, bk = digit_zeros(Kb)
    nq16, nk16 = -(-n // 16), -(-((T + 63) // 64 * 64) // 16)
    total = 0.0
    for h in range(H):
        if bq[h * n:(h + 1) * n].any() or bk[h * T:(h + 1) * T].any():
            continue
        q = np.full(nq16 * 16, 2, np.int32)
        q[:n] = zq[h * n:(h + 1) * n]
        k = np.full(nk16 * 16, 2, np.int32)
        k[:T] = zk[h * T:(h + 1) * T]
        a = float((5 - q.reshape(-1, 16).min(axis=1)).sum())
        b = float((5 - k.reshape(-1, 16).min(axis=1)).sum())
        i8 = (d // 64) * a * b * 32768.0
        waves = -(-n // 128) * 8
        bf16 = waves * ((T + 63) // 64) * (6 * d // 16) * 16384.0
        total += i8 + 2.0 * bf16
    return total


def source_hash(kernel: str) -> str:
    with open(KERNEL_SOURCES[kernel], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per launch of a kernel, measured by rocprofv3 counters, if they
    were taken on the kernel's current source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("traffic:"):
                continue
            vals = dict(kv.split("=") for kv in line[len("traffic:"):].split())
            if vals.get("kernel") != kernel:
                continue
            if vals.get("source_sha") != source_hash(kernel):
                return None
            try:
                return float(vals["bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


def status_bits(status: np.ndarray) -> dict:
    """Heads per head-status bit (the exact-refit marker included)."""
    names = ("chol_jitter", "nnls_cap", "nonfinite", "nnls_singular", "nnls_qr")
    return {nm: int(np.count_nonzero(status & (1 << i))) for i, nm in enumerate(names)
            if np.any(status & (1 << i))}


def cpu_baseline(idx: int, sample_heads: int):
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    w = synth.workload(idx)
    heads = w.heads(list(range(sample_heads)))
    t0 = time.perf_counter()
    for h, b in zip(heads, w.budgets[:sample_heads]):
        oracle.compact(h.Q, h.K, h.V, b, w.topk, w.refit_every)
    dt = time.perf_counter() - t0
    return {"value": sample_heads / dt, "unit": "heads/s", "cores": threads, "kind": "oracle",
            "sample": f"first {sample_heads} heads of the workload, float64 numpy/scipy oracle, {dt:.1f} s"}


def _online_round_bits(job):
    r, h = job
    w = synth.online_workload()
    head = w.initial([h])[0]
    budget = max(1, int(round((w.L - w.keep_newest) * w.ratio)))
    q, k, v = w.round_tokens(r, h, head.centres, w.L - budget - w.keep_newest)
    return synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(v)


def bench_online(args):
    """The online loop: every round compacts all 288 heads' prefixes (4076 keys
    to 2038, carrying beta from the rounds before) and refills the cache."""
    import torch

    from attention_matching_least_amd import amc, online

    dev = torch.device("cuda:0")
    w = synth.online_workload()
    H = w.num_heads
    t_gen = time.perf_counter()
    with ProcessPoolExecutor(max_workers=args.workers) as ex:
        heads_bits = list(ex.map(_online_init_bits, range(H), chunksize=4))
        rb = list(ex.map(_online_round_bits, [(r, h) for r in range(w.rounds) for h in range(H)], chunksize=4))
    gen_s = time.perf_counter() - t_gen

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    K0 = torch.stack([up(b[0]) for b in heads_bits])
    V0 = torch.stack([up(b[1]) for b in heads_bits])
    Qr = [torch.stack([up(rb[r * H + h][0]) for h in range(H)]) for r in range(w.rounds)]
    Kr = [torch.stack([up(rb[r * H + h][1]) for h in range(H)]) for r in range(w.rounds)]
    Vr = [torch.stack([up(rb[r * H + h][2]) for h in range(H)]) for r in range(w.rounds)]
    del rb, heads_bits
    timer = None if args.no_timer else amc.Timer()

    def run(tm):
        cache = online.Cache(K0, V0, torch.zeros((H, w.L), dtype=torch.float32, device=dev))
        return online.online_loop(cache, lambda r: Qr[r], lambda r, c: (Kr[r], Vr[r]), w.rounds,
                                  keep_newest=w.keep_newest, ratio=w.ratio, topk=w.topk,
                                  refit_every=w.refit_every, timer=tm)

    for _ in range(args.warmup):
        run(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = run(timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    status = np.concatenate([rd.result.head_status.cpu().numpy() for rd in out.rounds])
    kernels = timer.summary() if timer else {}
    print(json.dumps({
        "metric": "KV heads re-compacted/sec, online loop (T=4076 -> 2038 per round, d=128)",
        "value": round(H * w.rounds * args.steps / elapsed, 3),
        "unit": "heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000.0 * elapsed / args.steps, 1),
        "higher_is_better": True,
        "dtype": "f64",
        "data": "synthetic (seeded clustered Gaussians, bf16)",
        "config": {"workload": w.name, "heads": H, "L": w.L, "n": w.n, "d": w.d, "rounds": w.rounds,
                   "keep_newest": w.keep_newest, "ratio": w.ratio, "topk": w.topk,
                   "refit_every": w.refit_every},
        "kernels_ms": {k: round(v["total_ms"] / args.steps, 1) for k, v in kernels.items()},
        "head_status_nonzero": int(np.count_nonzero(status & ~amc.HS_NNLS_QR)),
        "head_status_bits": status_bits(status),
        "input_generation_s": round(gen_s, 1),
    }), flush=True)


SELECT_CLASSES = ("init", "shift", "phi", "sweep", "merge", "panel", "gram", "nnls", "resid")


def gen_long(args, H: int):
    """Inputs of the 60k-token stack (H heads), bf16 bit patterns per head.
    Generated in worker processes before anything touches the GPU."""
    flat = []
    with ProcessPoolExecutor(max_workers=args.workers) as ex:
        for g0 in range(0, H, 48):
            flat.extend(ex.map(_head_bits, [(3, h) for h in range(g0, min(H, g0 + 48))], chunksize=1))
            print(f"60k-token stack: generated heads up to {min(H, g0 + 48)}", file=sys.stderr, flush=True)
    return flat


def run_long(args, flat, H: int, timer=None):
    """Wall-clock seconds of the compaction calls over the 60k-token stack's H
    heads (key selection: shift, mass features, sweeps with Phi recomputed,
    panel, Gram, NNLS refits, residuals; plus the value fit and packing, so the
    figure bounds the key selection from above), in as few calls as the free
    device memory allows.  Returns the JSON fields of the measurement."""
    import torch

    from attention_matching_least_amd import amc

    dev = torch.device("cuda:0")
    w = synth.workload(3)
    if args.head_batch > 0:
        B = max(1, min(args.head_batch, H))
    else:
        # the fewest calls whose workspace and inputs fit in free memory, less 4 GB
        free = torch.cuda.mem_get_info(dev)[0] - (4 << 30)
        per_in = w.n * w.d * 2 + 2 * w.T * w.d * 2
        for ncall in range(1, H + 1):
            B = -(-H // ncall)
            need = amc.compact_workspace_bytes([w.n * h for h in range(B + 1)], [w.T * h for h in range(B + 1)],
                                               w.budgets[:B], w.d, select="batched", topk=w.topk,
                                               refit_every=w.refit_every, phi_budget_bytes=0)
            if need + B * per_in <= free:
                break
    allparts = [flat[b0:b0 + B] for b0 in range(0, H, B)]
    flat.clear()
    sel_ms, call_s, statuses, kern = 0.0, 0.0, [], {}
    for bi, b0 in enumerate(range(0, H, B)):
        hs = list(range(b0, min(H, b0 + B)))
        parts = allparts[bi]

        def up(k):
            a = np.concatenate([p[k] for p in parts])
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

        Q, K, V = up(0), up(1), up(2)
        allparts[bi] = parts = None
        nb = len(hs)
        cu_q = [w.n * h for h in range(nb + 1)]
        cu_k = [w.T * h for h in range(nb + 1)]
        # the whole stack's Phi (566 GB) is over the 64 GB budget, so each batch
        # runs as the whole call would: every sweep recomputes Phi
        kw = dict(cu_q=cu_q, cu_k=cu_k, select="batched", topk=w.topk, refit_every=w.refit_every,
                  phi_budget_bytes=0, head_groups=args.head_groups)
        if timer:
            timer.reset()
        torch.cuda.synchronize()
        print(f"60k-token stack: call {bi} on heads {hs[0]}..{hs[-1]}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        res = amc.compact(Q, K, V, w.budgets[b0:b0 + nb], timer=timer, **kw)
        torch.cuda.synchronize()
        call_s += time.perf_counter() - t0
        statuses.append(res.head_status.cpu().numpy())
        if timer:
            summ = timer.summary()
            sel_ms += sum(v["total_ms"] for k, v in summ.items() if k in SELECT_CLASSES)
            for k, v in summ.items():
                kern[k] = kern.get(k, 0.0) + v["total_ms"]
        del Q, K, V, res
        torch.cuda.empty_cache()
        print(f"60k-token stack: call {bi} done, {call_s:.1f} s so far", file=sys.stderr, flush=True)
    status = np.concatenate(statuses)
    scale = w.num_heads / H
    out = {
        "metric": "OMP key-select s at T=60k",
        "value": round(call_s * scale, 2),
        "value_covers": "wall-clock seconds of the compaction calls: key selection plus the value fit and packing",
        "parity": "the Gram-form refits' default entering test: in spot replays against the float64 oracle "
                  "the picks after refit 1 follow the oracle's, those after refit 12 of 47 do not (with "
                  "nnls_tol=1e-14 those after refits 12 and 24 do, at about 4x the time per head)",
        "unit": "s",
        "higher_is_better": False,
        "config": {"workload": w.name, "heads_run": H, "heads_total": w.num_heads, "head_batch": B, "T": w.T,
                   "n": w.n, "d": w.d, "budget": w.budgets[0], "topk": w.topk, "refit_every": w.refit_every,
                   "phi": "recomputed in every sweep"},
        "calls": len(allparts),
        "extrapolated_from_heads": H if H < w.num_heads else None,
        "full_call_s_measured": round(call_s, 3),
        "head_status_nonzero": int(np.count_nonzero(status & ~amc.HS_NNLS_QR)),
        "head_status_bits": status_bits(status),
        "heads_exact_refit": int(np.count_nonzero(status & 16)),
    }
    if timer:
        out["key_select_kernel_sum_s"] = round(sel_ms / 1e3, 3)
        out["kernels_ms_measured"] = {k: round(v, 1) for k, v in kern.items()}
    return out


def bench_long(args):
    """The 60k-token stack alone (--workload 3), with the per-kernel timer."""
    from attention_matching_least_amd import amc

    w = synth.workload(3)
    H = args.heads if args.heads > 0 else w.num_heads
    t_gen = time.perf_counter()
    flat = gen_long(args, H)
    gen_s = time.perf_counter() - t_gen
    timer = None if args.no_timer else amc.Timer()
    res = run_long(args, flat, H, timer)
    res.update({"n_gpus": 1, "steps": 1, "warmup": 0, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
                "data": "synthetic (seeded clustered Gaussians, bf16)", "input_generation_s": round(gen_s, 1)})
    print(json.dumps(res), flush=True)


def _online_init_bits(h):
    head = synth.online_workload().initial([h])[0]
    return synth.bf16_bits(head.K), synth.bf16_bits(head.V)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4],
                    help="1: one 8-head layer, plain OMP; 2: 288-head stack, batched selection; "
                         "3: 60k-token stack (wall-clock seconds of the compaction calls, Phi recomputed); "
                         "4: 288 heads with Dirichlet budgets 8..2048")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the peak probe (MFMA, vector f64 and HBM read rates of this GPU)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run three device-to-device copies of BYTES (the reference kernel for "
                         "scaling HBM byte counters)")
    ap.add_argument("--heads", type=int, default=0, help="workload 3: heads to run (0: all 288)")
    ap.add_argument("--head-batch", type=int, default=0,
                    help="workload 3: heads per compaction call (0: as many as free memory allows)")
    ap.add_argument("--cpu-sample", type=int, default=8, help="oracle heads timed for the CPU baseline (0: skip)")
    ap.add_argument("--no-long", action="store_true",
                    help="leave out the 60k-token stack's key-selection seconds (run by default with workload 2)")
    ap.add_argument("--workers", type=int, default=min(16, len(os.sched_getaffinity(0))))
    ap.add_argument("--exact-refit", default="auto", choices=["auto", "cold", "gated", "never"],
                    help="NNLS refits through the orthogonal factorisation: every head it takes, warm-started by "
                         "the Gram solver; every head it takes, warm-started by the previous refit; heads the "
                         "Gram solver flags; none")
    ap.add_argument("--nnls-tol", type=float, default=0.0,
                    help="the Gram solver's entering test relative to max |b| in every refit (0: the library's)")
    ap.add_argument("--no-highest", action="store_true", help="leave out the AM-Highest line")
    ap.add_argument("--recompute", action="store_true",
                    help="workloads 1, 2, 4: Phi recomputed in every sweep instead of stored (the mode the 60k-token "
                         "stack takes past its Phi budget), timed on the same inputs; no kernel pass or roofline")
    ap.add_argument("--no-timer", action="store_true", help="skip the kernel pass (per-kernel events, roofline)")
    ap.add_argument("--head-groups", type=int, default=0,
                    help="head groups (streams) of the timed steps; 0: the library's choice")
    ap.add_argument("--online", action="store_true",
                    help="time the online re-compaction loop (288 heads, 4096-token cache, 6 rounds of 50%%, "
                         "newest 20 kept) instead")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the heads of a call are independent, "
              "so a multi-GPU run would shard them by head with no collective on the hot path.", file=sys.stderr)
        sys.exit(2)

    if args.peaks:
        import subprocess

        probe = os.path.join(ROOT, "attention_matching_least_amd", "amc_peaks")
        if not os.path.exists(probe):
            sys.exit("amc_peaks is not built: run __graft_entry__.build() first")
        sys.exit(subprocess.run([probe]).returncode)

    import torch

    from attention_matching_least_amd import amc

    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "copies": 3}), flush=True)
        return
    if args.online:
        bench_online(args)
        return
    if args.workload == 3:
        bench_long(args)
        return
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w, Qb, Kb, Vb = generate(args.workload, args.workers)
    gen_s = time.perf_counter() - t_gen
    # the 60k-token stack's inputs too, before anything touches the GPU
    long_flat, long_H, long_gen_s = None, 0, 0.0
    if args.workload == 2 and not args.no_long:
        long_H = args.heads if args.heads > 0 else synth.workload(3).num_heads
        t_lg = time.perf_counter()
        long_flat = gen_long(args, long_H)
        long_gen_s = time.perf_counter() - t_lg
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    Q, K, V = up(Qb), up(Kb), up(Vb)
    phi_ops = phi_matrix_ops(Qb, Kb, w) if (w.dtype == "bf16" and not args.no_timer) else None
    del Qb, Kb, Vb
    H = w.num_heads
    cu_q = [w.n * h for h in range(H + 1)]
    cu_k = [w.T * h for h in range(H + 1)]
    select = "omp" if (w.topk == 1 and w.refit_every == 1) else "batched"
    kw = dict(cu_q=cu_q, cu_k=cu_k, select=select, topk=w.topk, refit_every=w.refit_every,
              exact_refit=args.exact_refit, nnls_tol=args.nnls_tol)
    if args.recompute:
        kw["phi_budget_bytes"] = 0
        args.no_timer = True
    ws_bytes = amc.compact_workspace_bytes(cu_q, cu_k, w.budgets, w.d, tdt, select=select, topk=w.topk,
                                           refit_every=w.refit_every, exact_refit=args.exact_refit,
                                           phi_budget_bytes=kw.get("phi_budget_bytes"))
    workspace = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    timer = None if args.no_timer else amc.Timer()

    for _ in range(args.warmup):
        amc.compact(Q, K, V, w.budgets, workspace=workspace, head_groups=args.head_groups, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = amc.compact(Q, K, V, w.budgets, workspace=workspace, head_groups=args.head_groups, **kw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    status = res.head_status.cpu().numpy()
    ms_per_step = 1000.0 * elapsed / args.steps
    value = H * args.steps / elapsed
    print(f"{w.name}: {args.steps} timed steps, {ms_per_step:.1f} ms per step", file=sys.stderr, flush=True)

    roofline = None
    roofline_other = None
    roofline_fit = None
    kernels = None
    kernel_pass = None
    if timer:
        # kernel pass: the same steps again with the heads in one group, so that
        # no two launches overlap and each event pair times one kernel alone
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            kres = amc.compact(Q, K, V, w.budgets, workspace=workspace, head_groups=1, timer=timer, trace=True,
                               **kw)
        torch.cuda.synchronize()
        print("kernel pass done", file=sys.stderr, flush=True)
        kernel_pass = {"head_groups": 1, "steps": args.steps,
                       "ms_per_step": round(1000.0 * (time.perf_counter() - t1) / args.steps, 3)}
        kernels = timer.summary()
        found = []
        kr = w.topk * w.refit_every
        sw = kernels.get("sweep")
        if sw:
            # algorithmic bytes: the stored high plane's columns of the keys each bounded
            # sweep reads (every key on the first cycle, the pruning's survivors after),
            # ldN = n rounded up to 64 queries of 2 bytes each, the 8-bit plane's columns
            # the second pruning stage reads (1 byte per query), and the 8-bit plane the
            # first cycle writes (every key), from the trace
            ldn = (w.n + 63) // 64 * 64
            ktr = kres.trace()
            swept = sum(int(c.sum()) for c in ktr["swept_keys"])
            swept8 = sum(int(c.sum()) for c in ktr["swept_keys8"])
            q8_written = H * w.T if swept8 > 0 else 0
            per_step = float(swept) * ldn * 2 + float(swept8 + q8_written) * ldn
            achieved = per_step * args.steps / (sw["total_ms"] * 1e-3) / 1e9
            found.append((sw["total_ms"], {
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("k_sweep"),
                "kernel": "k_sweep_band+k_sweep_q8", "avg_launch_ms": round(sw["avg_ms"], 4), "launches": sw["launches"],
                "algorithmic_bytes_per_launch": per_step * args.steps / sw["launches"],
                "swept_keys_per_step": swept, "swept_keys8_per_step": swept8,
                "keys_per_step_unpruned": int(sum(-(-b // kr) for b in w.budgets)) * w.T}))
        ph = kernels.get("phi")
        if ph:
            # algorithmic work of the mass features per head: Phi written (n T float32 values,
            # as its two 16-bit planes), Q, K, V read (bf16), m (float64) and Y (float32)
            # written; 2 n T d flops for Q K^T and 2 n T d for Phi V
            secs = ph["total_ms"] * 1e-3
            esz = 2 if w.dtype == "bf16" else 4
            bytes_head = 4.0 * w.n * w.T + esz * (w.n + 2 * w.T) * w.d + 8.0 * w.n + 4.0 * w.n * w.d
            per_step = bytes_head * H
            achieved = per_step * args.steps / secs / 1e9
            flops = 4.0 * w.n * w.T * w.d * H * args.steps
            found.append((ph["total_ms"], {
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("k_phi"),
                "kernel": "k_phi8", "avg_launch_ms": round(ph["avg_ms"], 4), "launches": ph["launches"],
                "algorithmic_bytes_per_launch": per_step * args.steps / ph["launches"],
                "bf16_mfma_tflops": round(flops / secs / 1e12, 2),
                "bf16_mfma_frac": round(flops / secs / 1e12 / BF16_MFMA_PEAK_TFS, 4),
                "int8_ops_executed_per_launch": (phi_ops * args.steps / ph["launches"]) if phi_ops else None,
                "int8_ops_frac": round(phi_ops * args.steps / secs / 1e12 / I8_MFMA_PEAK_TOPS, 4) if phi_ops else None}))
        found.sort(key=lambda x: -x[0])
        if found:
            roofline = found[0][1]
        if len(found) > 1:
            roofline_other = found[1][1]
        # the float64 matrix-core contractions of the fit side, by the method's flops
        # (each head alike; a padded tile counts only its rows and columns in use):
        # the Gram update of cycle c is [panel rows S0 + Kc, m] x [Kc new keys, r]
        # over the n queries (the polish refit: the panel rows by r); the value fit's
        # normal equations N = A^T A (one triangle) and A^T Y
        # (the Gram update reads the panel rows, m, r and the new keys' rows once per
        # cycle: its bytes against the HBM roof too)
        fit_flops, gram_bytes = {}, 0.0
        for b in w.budgets:
            gram = 0.0
            for c in range(-(-b // kr)):
                s0 = c * kr
                kc = min(kr, b - s0)
                gram += 2.0 * w.n * (s0 + kc + 1) * (kc + 1)
                gram_bytes += 8.0 * w.n * (s0 + 2 * kc + 2)
            gram += 2.0 * w.n * b
            gram_bytes += 8.0 * w.n * (b + 1)
            fit_flops["gram"] = fit_flops.get("gram", 0.0) + gram
            fit_flops["ols_normal"] = fit_flops.get("ols_normal", 0.0) + 2.0 * w.n * (b * (b + 1) / 2 + b * w.d)
        roofline_fit = {}
        for cls, kname in (("gram", "k_gram"), ("ols_normal", "k_ols_normal")):
            kk = kernels.get(cls)
            if kk and kk["total_ms"] > 0:
                tf = fit_flops[cls] * args.steps / (kk["total_ms"] * 1e-3) / 1e12
                roofline_fit[kname] = {"bound": "mfma", "achieved": round(tf, 2), "peak": F64_MFMA_PEAK_TFS,
                                       "unit": "TFLOP/s", "frac": round(tf / F64_MFMA_PEAK_TFS, 4),
                                       "flops_per_step": fit_flops[cls], "avg_launch_ms": round(kk["avg_ms"], 4),
                                       "launches": kk["launches"]}
                if cls == "gram":
                    gbs = gram_bytes * args.steps / (kk["total_ms"] * 1e-3) / 1e9
                    roofline_fit[kname].update({"bytes_per_step": gram_bytes, "hbm_gbs": round(gbs, 1),
                                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})

    highest = None
    if not args.no_highest:
        # AM-Highest on the same resident inputs (one scoring sweep, top t, one
        # refit, the value fit): the method family's fast member, beside the metric
        ws_h = amc.compact_workspace_bytes(cu_q, cu_k, w.budgets, w.d, tdt, select="highest")
        if ws_h + 256 > workspace.numel():
            workspace = torch.empty(ws_h + 256, dtype=torch.uint8, device=dev)
        kh = dict(cu_q=cu_q, cu_k=cu_k, select="highest", exact_refit=args.exact_refit)
        for _ in range(args.warmup):
            amc.compact(Q, K, V, w.budgets, workspace=workspace, head_groups=args.head_groups, **kh)
        torch.cuda.synchronize()
        th = time.perf_counter()
        for _ in range(args.steps):
            hres = amc.compact(Q, K, V, w.budgets, workspace=workspace, head_groups=args.head_groups, **kh)
        torch.cuda.synchronize()
        hsec = time.perf_counter() - th
        hstat = hres.head_status.cpu().numpy()
        print(f"AM-Highest: {1000.0 * hsec / args.steps:.1f} ms per step", file=sys.stderr, flush=True)
        highest = {"select": "AM-Highest", "value": round(H * args.steps / hsec, 2), "unit": "heads/s",
                   "ms_per_step": round(1000.0 * hsec / args.steps, 3),
                   "heads_exact_refit": int(np.count_nonzero(hstat & 16))}
        del hres

    cpu = cpu_baseline(args.workload, args.cpu_sample) if args.cpu_sample > 0 else None
    if cpu:
        print(f"CPU oracle: {cpu['value']:.3f} heads/s", file=sys.stderr, flush=True)
    long_ctx = None
    if long_flat is not None:
        # the headline's buffers go before the 60k-token stack takes the card
        del Q, K, V, workspace, res
        if timer:
            del kres
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        long_ctx = run_long(args, long_flat, long_H)
        long_ctx["input_generation_s"] = round(long_gen_s, 1)

    out = {
        "metric": "KV heads compacted/sec at T=8192,50x (d=128)",
        "value": round(value, 2),
        "unit": "heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded clustered Gaussians, bf16)",
        "config": {"workload": w.name, "heads": H, "T": w.T, "n": w.n, "d": w.d,
                   "budget": w.budgets[0] if len(set(w.budgets)) == 1 else
                   f"{min(w.budgets)}..{max(w.budgets)} (sum {sum(w.budgets)})",
                   "topk": w.topk, "refit_every": w.refit_every, "parallelism": "none (one GPU)",
                   "phi": "recomputed in every sweep" if args.recompute else "stored (two 16-bit planes)"},
        "roofline": roofline,
        "roofline_next": roofline_other,
        "roofline_fit": roofline_fit,
        "cpu_baseline": cpu,
        "kernel_pass": kernel_pass,
        "kernels_ms": {k: round(v["total_ms"] / args.steps, 3) for k, v in (kernels or {}).items()},
        "head_status_nonzero": int(np.count_nonzero(status & ~amc.HS_NNLS_QR)),
        "head_status_bits": status_bits(status),
        "heads_exact_refit": int(np.count_nonzero(status & 16)),
        "input_generation_s": round(gen_s, 1),
        "long_context": long_ctx,
        "highest": highest,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
