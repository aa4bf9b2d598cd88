"""Python binding of libamc (ctypes).

Argument marshalling only: every step of the compaction runs in the HIP
library.  PyTorch supplies device memory (outputs, workspace, trace) and the
current HIP stream.  The binding fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libamc.so")

AMC_OK, AMC_ERR_INVALID_ARG, AMC_ERR_UNSUPPORTED, AMC_ERR_WORKSPACE, AMC_ERR_HIP = 0, 1, 2, 3, 4
AMC_F32, AMC_BF16 = 0, 1
AMC_SEL_OMP, AMC_SEL_OMP_BATCHED, AMC_SEL_HIGHEST = 0, 1, 2
AMC_FLAG_TRACE = 1
HS_CHOL_JITTER, HS_NNLS_CAP, HS_NONFINITE, HS_NNLS_SINGULAR, HS_NNLS_QR = 1, 2, 4, 8, 16
EXACT_REFIT = {"auto": 3, "cold": 0, "gated": 1, "never": 2}

KERNEL_CLASSES = ["init", "shift", "phi", "sweep", "merge", "panel", "gram", "nnls", "resid",
                  "ols_normal", "ols_solve", "pack", "sweep_exact", "rescore", "prune", "digits", "phi_f64"]

EXPORTED = [
    "amc_default_options", "amc_workspace_size", "amc_output_offsets", "amc_cycle_offsets",
    "amc_trace_layout_for", "amc_compact", "amc_mass_features", "amc_mass_features_workspace", "amc_nnls",
    "amc_timer_create", "amc_timer_reset", "amc_timer_read", "amc_timer_destroy", "amc_status_string",
    "amc_version", "amc_compact_noalloc", "amc_noalloc_max_workspace", "amc_greedy_swap_budgets",
]


class AmcError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cu_q", ctypes.c_void_p),
        ("cu_k", ctypes.c_void_p),
        ("budgets", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class Options(ctypes.Structure):
    _fields_ = [
        ("select", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("refit_every", ctypes.c_int32),
        ("nnls_max_iters", ctypes.c_int32),
        ("nnls_polish", ctypes.c_int32),
        ("nnls_tol", ctypes.c_double),
        ("phi_budget_bytes", ctypes.c_uint64),
        ("cv_dtype", ctypes.c_int32),
        ("head_groups", ctypes.c_int32),
        ("exact_refit", ctypes.c_int32),
        ("digits_in_panel", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("timer", ctypes.c_void_p),
    ]


class TraceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("shift", "pick", "pick_score", "weight", "runner_up", "nnls_iters", "swept_keys",
                 "swept_keys8", "relres", "total_bytes")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libamc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libamc.so not found at {LIB_PATH}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    P, O = ctypes.POINTER(Problem), ctypes.POINTER(Options)
    L.amc_default_options.argtypes = [O]
    L.amc_default_options.restype = None
    L.amc_workspace_size.argtypes = [P, O, ctypes.POINTER(u64)]
    L.amc_output_offsets.argtypes = [P, ctypes.POINTER(i64)]
    L.amc_cycle_offsets.argtypes = [P, O, ctypes.POINTER(i64)]
    L.amc_trace_layout_for.argtypes = [P, O, ctypes.POINTER(TraceLayout)]
    L.amc_compact.argtypes = [P, O, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, vp, u64, vp]
    L.amc_compact_noalloc.argtypes = [P, O, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, vp]
    L.amc_noalloc_max_workspace.argtypes = []
    L.amc_noalloc_max_workspace.restype = u64
    L.amc_mass_features.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, vp]
    L.amc_mass_features_workspace.argtypes = [P, ctypes.POINTER(u64)]
    L.amc_nnls.argtypes = [i32, ctypes.POINTER(i64), vp, vp, vp, i32, i32, i32, dbl, vp, vp, vp]
    L.amc_greedy_swap_budgets.argtypes = [i32, i32, vp, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.amc_timer_create.argtypes = [ctypes.POINTER(vp)]
    L.amc_timer_reset.argtypes = [vp]
    L.amc_timer_read.argtypes = [vp, i32, ctypes.POINTER(i64), ctypes.POINTER(dbl)]
    L.amc_timer_destroy.argtypes = [vp]
    L.amc_timer_destroy.restype = None
    L.amc_status_string.argtypes = [i32]
    L.amc_status_string.restype = ctypes.c_char_p
    L.amc_version.restype = ctypes.c_int
    for name in ("amc_workspace_size", "amc_output_offsets", "amc_cycle_offsets", "amc_trace_layout_for",
                 "amc_compact", "amc_compact_noalloc", "amc_mass_features", "amc_mass_features_workspace", "amc_nnls",
                 "amc_greedy_swap_budgets",
                 "amc_timer_create", "amc_timer_reset", "amc_timer_read"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(s: int) -> str:
    try:
        return lib().amc_status_string(int(s)).decode()
    except Exception:  # pragma: no cover - library missing
        return "unknown"


def _check(st: int, what: str):
    if st != AMC_OK:
        raise AmcError(st, what)


def version() -> int:
    return int(lib().amc_version())


# ----------------------------------------------------------------------------
# argument marshalling
# ----------------------------------------------------------------------------
def _i64_array(values: Sequence[int]):
    arr = (ctypes.c_int64 * len(values))(*[int(v) for v in values])
    return arr


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return AMC_BF16
    if t.dtype == torch.float32:
        return AMC_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _as_packed(x: torch.Tensor, cu: Optional[Sequence[int]], name: str):
    """(H, n, d) -> (H*n, d) and offsets; (N, d) + offsets -> unchanged."""
    if x.dim() == 3:
        H, n, d = x.shape
        return x.reshape(H * n, d), [n * h for h in range(H + 1)]
    if x.dim() == 2:
        if cu is None:
            raise ValueError(f"{name}: packed 2-D input needs its row offsets")
        return x, [int(v) for v in cu]
    raise ValueError(f"{name}: expected a 2-D packed or 3-D (heads, rows, dim) tensor")


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _aligned_workspace(nbytes: int, device) -> (torch.Tensor, int):
    buf = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    ptr = buf.data_ptr()
    return buf, (ptr + 255) // 256 * 256


def make_problem(num_heads: int, head_dim: int, cu_q: Sequence[int], cu_k: Sequence[int],
                 budgets: Sequence[int], in_dtype: int, scale: float = 0.0):
    """A Problem struct plus the ctypes arrays it points to (kept alive together)."""
    aq, ak, ab = _i64_array(cu_q), _i64_array(cu_k), _i64_array(budgets)
    p = Problem(int(num_heads), int(head_dim), ctypes.cast(aq, ctypes.c_void_p), ctypes.cast(ak, ctypes.c_void_p),
                ctypes.cast(ab, ctypes.c_void_p), int(in_dtype), float(scale))
    return p, (aq, ak, ab)


def make_options(select: str = "omp", topk: int = 1, refit_every: int = 1, nnls_polish: int = 1,
                 nnls_max_iters: int = 0, nnls_tol: float = 0.0, phi_budget_bytes: Optional[int] = None,
                 cv_dtype: torch.dtype = torch.float32, trace: bool = False, timer: "Timer" = None,
                 head_groups: int = 0, exact_refit: str = "auto", digits_in_panel: bool = True) -> Options:
    o = Options()
    lib().amc_default_options(ctypes.byref(o))
    o.select = {"omp": AMC_SEL_OMP, "batched": AMC_SEL_OMP_BATCHED, "highest": AMC_SEL_HIGHEST}[select]
    o.topk = int(topk)
    o.refit_every = int(refit_every)
    o.nnls_polish = int(nnls_polish)
    o.nnls_max_iters = int(nnls_max_iters)
    o.nnls_tol = float(nnls_tol)
    if phi_budget_bytes is not None:
        o.phi_budget_bytes = int(phi_budget_bytes)
    o.cv_dtype = AMC_BF16 if cv_dtype == torch.bfloat16 else AMC_F32
    o.flags = AMC_FLAG_TRACE if trace else 0
    o.head_groups = int(head_groups)
    o.exact_refit = EXACT_REFIT[exact_refit]
    o.digits_in_panel = 1 if digits_in_panel else 0
    o.timer = timer.handle if timer is not None else None
    return o


def workspace_size(problem: Problem, options: Options) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().amc_workspace_size(ctypes.byref(problem), ctypes.byref(options), ctypes.byref(out)),
           "amc_workspace_size")
    return int(out.value)


def output_offsets(problem: Problem) -> List[int]:
    H = problem.num_heads
    arr = (ctypes.c_int64 * (H + 1))()
    _check(lib().amc_output_offsets(ctypes.byref(problem), arr), "amc_output_offsets")
    return list(arr)


def cycle_offsets(problem: Problem, options: Options) -> List[int]:
    H = problem.num_heads
    arr = (ctypes.c_int64 * (H + 1))()
    _check(lib().amc_cycle_offsets(ctypes.byref(problem), ctypes.byref(options), arr), "amc_cycle_offsets")
    return list(arr)


def trace_layout(problem: Problem, options: Options) -> TraceLayout:
    L = TraceLayout()
    _check(lib().amc_trace_layout_for(ctypes.byref(problem), ctypes.byref(options), ctypes.byref(L)),
           "amc_trace_layout_for")
    return L


# ----------------------------------------------------------------------------
# timer
# ----------------------------------------------------------------------------
class Timer:
    """HIP-event timer of libamc's kernel launches (per kernel class)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().amc_timer_create(ctypes.byref(h)), "amc_timer_create")
        self.handle = h.value

    def reset(self):
        _check(lib().amc_timer_reset(self.handle), "amc_timer_reset")

    def read(self, cls) -> (int, float):
        idx = KERNEL_CLASSES.index(cls) if isinstance(cls, str) else int(cls)
        n = ctypes.c_int64(0)
        ms = ctypes.c_double(0.0)
        _check(lib().amc_timer_read(self.handle, idx, ctypes.byref(n), ctypes.byref(ms)), "amc_timer_read")
        return int(n.value), float(ms.value)

    def summary(self) -> Dict[str, dict]:
        out = {}
        for c in KERNEL_CLASSES:
            n, ms = self.read(c)
            if n:
                out[c] = {"launches": n, "total_ms": ms, "avg_ms": ms / n}
        return out

    def close(self):
        if self.handle:
            lib().amc_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
@dataclass
class CompactResult:
    Ck: torch.Tensor  # [sum t][d] input dtype
    beta: torch.Tensor  # [sum t] float32
    Cv: torch.Tensor  # [sum t][d]
    sel_idx: torch.Tensor  # [sum t] int32
    cu_budgets: List[int]
    head_status: torch.Tensor  # [H] int32
    trace_buf: Optional[torch.Tensor] = None
    trace_layout: Optional[TraceLayout] = None
    cu_cycles: Optional[List[int]] = None
    num_heads: int = 0

    def head(self, h: int):
        a, b = self.cu_budgets[h], self.cu_budgets[h + 1]
        return self.Ck[a:b], self.beta[a:b], self.Cv[a:b], self.sel_idx[a:b]

    def trace(self) -> Dict[str, list]:
        """Per-head trace arrays (host numpy), after the stream has been synchronised."""
        if self.trace_buf is None:
            raise ValueError("compaction ran without trace=True")
        raw = self.trace_buf.cpu().numpy()
        L = self.trace_layout
        H = self.num_heads
        st = self.cu_budgets[-1]
        sc = self.cu_cycles[-1]

        def sec(off, dtype, count):
            return np.frombuffer(raw[off: off + np.dtype(dtype).itemsize * count].tobytes(), dtype=dtype)

        shift = sec(L.shift, np.float64, H)
        pick = sec(L.pick, np.int32, st)
        pick_score = sec(L.pick_score, np.float64, st)
        weight = sec(L.weight, np.float64, st)
        runner = sec(L.runner_up, np.float64, sc)
        iters = sec(L.nnls_iters, np.int32, sc)
        swept = sec(L.swept_keys, np.int32, sc)
        swept8 = sec(L.swept_keys8, np.int32, sc)
        relres = sec(L.relres, np.float64, sc)
        cb, cc = self.cu_budgets, self.cu_cycles
        return {
            "shift": shift,
            "pick": [pick[cb[h]:cb[h + 1]] for h in range(H)],
            "pick_score": [pick_score[cb[h]:cb[h + 1]] for h in range(H)],
            "weight": [weight[cb[h]:cb[h + 1]] for h in range(H)],
            "runner_up": [runner[cc[h]:cc[h + 1]] for h in range(H)],
            "nnls_iters": [iters[cc[h]:cc[h + 1]] for h in range(H)],
            "swept_keys": [swept[cc[h]:cc[h + 1]] for h in range(H)],
            "swept_keys8": [swept8[cc[h]:cc[h + 1]] for h in range(H)],
            "relres": [relres[cc[h]:cc[h + 1]] for h in range(H)],
        }


def compact(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, budgets, *, cu_q=None, cu_k=None,
            beta_in: Optional[torch.Tensor] = None, select: str = "omp", topk: int = 1, refit_every: int = 1,
            nnls_polish: int = 1, nnls_max_iters: int = 0, nnls_tol: float = 0.0,
            phi_budget_bytes: Optional[int] = None, cv_dtype: torch.dtype = torch.float32, trace: bool = False,
            timer: Optional[Timer] = None, scale: float = 0.0, stream=None,
            workspace: Optional[torch.Tensor] = None, head_groups: int = 0, exact_refit: str = "auto",
            digits_in_panel: bool = True, noalloc: bool = False) -> CompactResult:
    """amc_compact on torch tensors.  Q: (H, n, d) or packed (sum n, d) with
    cu_q; K, V: (H, T, d) or packed with cu_k; budgets: int or per-head list.
    noalloc: amc_compact_noalloc (the library's static per-GPU workspace; no
    workspace tensor is allocated here)."""
    if not (Q.is_cuda and K.is_cuda and V.is_cuda):
        raise ValueError("Q, K and V must be device tensors")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K and V must share one dtype")
    Qp, cq = _as_packed(Q, cu_q, "Q")
    Kp, ck = _as_packed(K, cu_k, "K")
    Vp, ck2 = _as_packed(V, cu_k, "V")
    if ck != ck2 or Kp.shape != Vp.shape or Qp.shape[1] != Kp.shape[1]:
        raise ValueError("K and V must have the same packing and Q, K the same head_dim")
    Qp, Kp, Vp = Qp.contiguous(), Kp.contiguous(), Vp.contiguous()
    H = len(cq) - 1
    d = int(Qp.shape[1])
    bud = [int(budgets)] * H if isinstance(budgets, (int, np.integer)) else [int(b) for b in budgets]
    if len(bud) != H:
        raise ValueError("one budget per head")
    prob, keep = make_problem(H, d, cq, ck, bud, _dtype_code(Qp), scale)
    opts = make_options(select, topk, refit_every, nnls_polish, nnls_max_iters, nnls_tol, phi_budget_bytes,
                        cv_dtype, trace, timer, head_groups, exact_refit, digits_in_panel)
    ws_bytes = 0 if noalloc else workspace_size(prob, opts)
    cb = output_offsets(prob)
    dev = Qp.device
    S = cb[-1]
    Ck = torch.empty((S, d), dtype=Qp.dtype, device=dev)
    beta = torch.empty(S, dtype=torch.float32, device=dev)
    Cv = torch.empty((S, d), dtype=cv_dtype, device=dev)
    sel = torch.empty(S, dtype=torch.int32, device=dev)
    hs = torch.empty(H, dtype=torch.int32, device=dev)
    if noalloc:
        ws_buf, ws_ptr = None, None
    elif workspace is not None and workspace.numel() >= ws_bytes + 256:
        ws_buf = workspace
        ws_ptr = (workspace.data_ptr() + 255) // 256 * 256
    else:
        ws_buf, ws_ptr = _aligned_workspace(ws_bytes, dev)
    tr_buf, tr_ptr, tl, cc = None, None, None, None
    tr_bytes = 0
    if trace:
        tl = trace_layout(prob, opts)
        tr_bytes = int(tl.total_bytes)
        tr_buf, tr_ptr = _aligned_workspace(tr_bytes, dev)
        cc = cycle_offsets(prob, opts)
    if beta_in is not None:
        if beta_in.dtype != torch.float32 or beta_in.numel() != ck[-1] or not beta_in.is_cuda:
            raise ValueError("beta_in must be a float32 device tensor with one entry per key")
        beta_in = beta_in.contiguous()
    bi_ptr = beta_in.data_ptr() if beta_in is not None else None
    if noalloc:
        st = lib().amc_compact_noalloc(ctypes.byref(prob), ctypes.byref(opts), Qp.data_ptr(), Kp.data_ptr(),
                                       Vp.data_ptr(), bi_ptr, Ck.data_ptr(), beta.data_ptr(), Cv.data_ptr(),
                                       sel.data_ptr(), hs.data_ptr(), tr_ptr, tr_bytes, _stream_ptr(stream))
        _check(st, "amc_compact_noalloc")
    else:
        st = lib().amc_compact(ctypes.byref(prob), ctypes.byref(opts), Qp.data_ptr(), Kp.data_ptr(), Vp.data_ptr(),
                               bi_ptr, Ck.data_ptr(), beta.data_ptr(), Cv.data_ptr(), sel.data_ptr(), hs.data_ptr(),
                               tr_ptr, tr_bytes, ws_ptr, ws_bytes, _stream_ptr(stream))
        _check(st, "amc_compact")
    res = CompactResult(Ck, beta, Cv, sel, cb, hs, None, tl, cc, H)
    if trace:
        # view of the aligned trace region
        off = tr_ptr - tr_buf.data_ptr()
        res.trace_buf = tr_buf[off: off + tr_bytes]
    res._keep = (ws_buf, tr_buf, keep)
    return res


def noalloc_max_workspace() -> int:
    """Bytes of the static per-GPU workspace of amc_compact_noalloc."""
    return int(lib().amc_noalloc_max_workspace())


def chunk_split(T: int, t: int, chunk_keys: int) -> List[tuple]:
    """The chunks [c L, min((c+1) L, T)) of L = chunk_keys keys and their
    budgets: t shared in proportion to the chunks' lengths by largest
    remainders (ties to the earlier chunk), each at least 1 and at most its
    length.  Returns [(k0, k1, t_c)]."""
    if not (1 <= t <= T) or chunk_keys < 1:
        raise ValueError("need 1 <= t <= T and chunk_keys >= 1")
    bounds = [(k0, min(k0 + chunk_keys, T)) for k0 in range(0, T, chunk_keys)]
    if t < len(bounds):
        raise ValueError("budget below one key per chunk")
    # exact rational quotas t * len / T as integer floor and remainder
    floors = [t * (k1 - k0) // T for k0, k1 in bounds]
    rems = [t * (k1 - k0) % T for k0, k1 in bounds]
    tc = [max(1, min(k1 - k0, f)) for (k0, k1), f in zip(bounds, floors)]
    left = t - sum(tc)
    order = sorted(range(len(bounds)), key=lambda c: (-rems[c], c))
    while left != 0:
        moved = False
        for c in order:
            k0, k1 = bounds[c]
            if left > 0 and tc[c] < k1 - k0:
                tc[c] += 1
                left -= 1
                moved = True
            elif left < 0 and tc[c] > 1:
                tc[c] -= 1
                left += 1
                moved = True
            if left == 0:
                break
        if not moved:
            raise ValueError("no feasible split")
    return [(k0, k1, c) for (k0, k1), c in zip(bounds, tc)]


@dataclass
class ChunkedResult:
    """amc_compact over the chunks of every head (each chunk a head of its own),
    in each head's output range.  sel_idx counts keys within the original head."""
    result: CompactResult  # per chunk-head outputs and trace
    split: List[List[tuple]]  # per original head: (k0, k1, t_c) of each chunk
    cu_budgets: List[int]
    sel_idx: torch.Tensor

    def head(self, h: int):
        a, b = self.cu_budgets[h], self.cu_budgets[h + 1]
        r = self.result
        return r.Ck[a:b], r.beta[a:b], r.Cv[a:b], self.sel_idx[a:b]

    def chunk_head(self, h: int, c: int) -> int:
        """Index of head h's chunk c among the chunk-heads of the call."""
        return sum(len(s) for s in self.split[:h]) + c


def compact_chunked(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, budgets, chunk_keys: int, *, cu_q=None,
                    cu_k=None, beta_in: Optional[torch.Tensor] = None, **kw) -> ChunkedResult:
    """KV-based chunked compaction (xinfinite.net article, section 3, chunked
    compression; zhichai.net deep-dive, section 4.3): every head's keys are cut
    into chunks of chunk_keys consecutive keys, each chunk is compacted as a
    head of its own against the head's reference queries (budget shared by
    chunk_split), and the compacted chunks stay in key order in the head's
    output range.  One amc_compact call: the chunks' keys, values and bias
    are the caller's rows as they are; each chunk-head gets its own copy of
    the head's query rows.  Other arguments as for compact()."""
    Qp, cq = _as_packed(Q, cu_q, "Q")
    Kp, ck = _as_packed(K, cu_k, "K")
    Vp, _ = _as_packed(V, cu_k, "V")
    H = len(cq) - 1
    tb = [int(budgets)] * H if isinstance(budgets, int) else [int(b) for b in budgets]
    split, rows, cq2, ck2, b2, off = [], [], [0], [0], [], []
    for h in range(H):
        sp = chunk_split(ck[h + 1] - ck[h], tb[h], chunk_keys)
        split.append(sp)
        n = cq[h + 1] - cq[h]
        for k0, k1, tc in sp:
            rows.append(torch.arange(cq[h], cq[h + 1], device=Qp.device))
            cq2.append(cq2[-1] + n)
            ck2.append(ck[h] + k1)
            b2.append(tc)
            off.extend([k0] * tc)
    Q2 = Qp.index_select(0, torch.cat(rows)).contiguous()
    res = compact(Q2, Kp, Vp, b2, cu_q=cq2, cu_k=ck2, beta_in=beta_in, **kw)
    sel = res.sel_idx + torch.tensor(off, dtype=torch.int32, device=res.sel_idx.device)
    cub = [0]
    for b in tb:
        cub.append(cub[-1] + b)
    return ChunkedResult(res, split, cub, sel)


def greedy_swap_budgets(loss, unit: int, total: int):
    """amc_greedy_swap_budgets: per-head budgets (keys) from sensitivity curves
    loss[h][j] (head h keeping (j+1) * unit keys) summing to total; returns
    (budgets, moves)."""
    L = np.ascontiguousarray(np.asarray(loss, dtype=np.float64))
    H, J = L.shape
    out = (ctypes.c_int64 * H)()
    mv = ctypes.c_int64(0)
    _check(lib().amc_greedy_swap_budgets(H, J, L.ctypes.data_as(ctypes.c_void_p), int(unit), int(total), out,
                                         ctypes.byref(mv)), "amc_greedy_swap_budgets")
    return [int(x) for x in out], int(mv.value)


def compact_workspace_bytes(cu_q, cu_k, budgets, head_dim: int, dtype: torch.dtype = torch.bfloat16,
                            **opt_kwargs) -> int:
    prob, keep = make_problem(len(cu_q) - 1, head_dim, cu_q, cu_k, budgets,
                              AMC_BF16 if dtype == torch.bfloat16 else AMC_F32)
    return workspace_size(prob, make_options(**opt_kwargs))


def mass_features(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, *, cu_q=None, cu_k=None,
                  beta_in: Optional[torch.Tensor] = None, want_phi: bool = True, scale: float = 0.0, stream=None):
    """amc_mass_features: (shift [H] f64, phi [sum n*T] f32 or None, m [sum n] f64, Y [sum n][d] f32, status)."""
    Qp, cq = _as_packed(Q, cu_q, "Q")
    Kp, ck = _as_packed(K, cu_k, "K")
    Vp, _ = _as_packed(V, cu_k, "V")
    Qp, Kp, Vp = Qp.contiguous(), Kp.contiguous(), Vp.contiguous()
    H = len(cq) - 1
    d = int(Qp.shape[1])
    prob, keep = make_problem(H, d, cq, ck, [1] * H, _dtype_code(Qp), scale)
    out = ctypes.c_uint64(0)
    _check(lib().amc_mass_features_workspace(ctypes.byref(prob), ctypes.byref(out)), "amc_mass_features_workspace")
    dev = Qp.device
    ws_buf, ws_ptr = _aligned_workspace(int(out.value), dev)
    n_tot = cq[-1]
    phi_elems = sum((cq[h + 1] - cq[h]) * (ck[h + 1] - ck[h]) for h in range(H))
    shift = torch.empty(H, dtype=torch.float64, device=dev)
    phi = torch.empty(phi_elems, dtype=torch.float32, device=dev) if want_phi else None
    m = torch.empty(n_tot, dtype=torch.float64, device=dev)
    Y = torch.empty((n_tot, d), dtype=torch.float32, device=dev)
    hs = torch.empty(H, dtype=torch.int32, device=dev)
    st = lib().amc_mass_features(ctypes.byref(prob), Qp.data_ptr(), Kp.data_ptr(), Vp.data_ptr(),
                                 beta_in.contiguous().data_ptr() if beta_in is not None else None,
                                 shift.data_ptr(), phi.data_ptr() if phi is not None else None, m.data_ptr(),
                                 Y.data_ptr(), hs.data_ptr(), ws_ptr, int(out.value), _stream_ptr(stream))
    _check(st, "amc_mass_features")
    (torch.cuda.current_stream() if stream is None else stream).synchronize()
    del ws_buf
    return shift, phi, m, Y, hs


def nnls(G_list: Sequence[np.ndarray], b_list: Sequence[np.ndarray], *, w0: Optional[Sequence[np.ndarray]] = None,
         pg_iters: int = 8, max_iters: int = 0, tol: float = 0.0, device="cuda"):
    """amc_nnls on host float64 systems; returns (list of w, iterations, status)."""
    ts = [int(np.asarray(b).shape[0]) for b in b_list]
    cu = [0]
    for t in ts:
        cu.append(cu[-1] + t)
    Gcat = np.concatenate([np.ascontiguousarray(G, dtype=np.float64).ravel() for G in G_list])
    bcat = np.concatenate([np.asarray(b, dtype=np.float64) for b in b_list])
    wcat = np.concatenate([np.asarray(w, dtype=np.float64) for w in w0]) if w0 is not None else np.zeros(cu[-1])
    Gd = torch.from_numpy(Gcat).to(device)
    bd = torch.from_numpy(bcat).to(device)
    wd = torch.from_numpy(wcat).to(device)
    num = len(ts)
    it = torch.empty(num, dtype=torch.int32, device=device)
    stt = torch.empty(num, dtype=torch.int32, device=device)
    arr = _i64_array(cu)
    st = lib().amc_nnls(num, arr, Gd.data_ptr(), bd.data_ptr(), wd.data_ptr(), 1 if w0 is not None else 0,
                        int(pg_iters), int(max_iters), float(tol), it.data_ptr(), stt.data_ptr(),
                        _stream_ptr(None))
    _check(st, "amc_nnls")
    torch.cuda.synchronize()
    w = wd.cpu().numpy()
    return [w[cu[i]:cu[i + 1]] for i in range(num)], it.cpu().numpy(), stt.cpu().numpy()
