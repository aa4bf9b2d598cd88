"""The C-ABI library: it loads, exports every symbol include/amc.h declares,
and rejects invalid arguments before touching the GPU (no device needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_matching_least_amd import amc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "amc.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(amc_[a-z0-9_]+)\s*\(", text)))


def _exported():
    out = subprocess.run(["nm", "-D", "--defined-only", amc.LIB_PATH], capture_output=True, text=True, check=True)
    return {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}


def test_library_loads_and_reports_version():
    assert amc.version() == 1


def test_every_declared_symbol_is_exported():
    declared = _declared_functions()
    assert len(declared) >= 14
    exported = _exported()
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert set(amc.EXPORTED) == set(declared)


def _problem(H=2, d=128, n=(100, 50), T=(300, 200), t=(10, 5), dtype=amc.AMC_BF16):
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(n, T):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    return amc.make_problem(H, d, cu_q, cu_k, list(t), dtype)


def test_default_options():
    o = amc.make_options()
    assert o.select == amc.AMC_SEL_OMP and o.topk == 1 and o.refit_every == 1
    assert o.phi_budget_bytes == 64 << 30
    assert o.nnls_polish == 1 and o.flags == 0


def test_offsets_and_workspace():
    p, keep = _problem()
    assert amc.output_offsets(p) == [0, 10, 15]
    o = amc.make_options(select="batched", topk=4, refit_every=2)
    assert amc.cycle_offsets(p, o) == [0, 2, 3]
    ws = amc.workspace_size(p, o)
    # at least Phi (float32) + panel (float64) + Gram (float64)
    assert ws >= 4 * (100 * 300 + 50 * 200) + 8 * (10 * 100 + 5 * 50) + 8 * (100 + 25)
    assert ws % 256 == 0
    L = amc.trace_layout(p, o)
    assert L.total_bytes >= 8 * 2 + 4 * 15 + 8 * 15 * 2 + 8 * 3 + 4 * 3
    assert all(getattr(L, f) % 256 == 0 for f in ("shift", "pick", "pick_score", "weight", "runner_up", "nnls_iters"))


def _status(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("bad", [
    dict(d=96),           # head_dim unsupported
    dict(t=(0, 5)),       # zero budget
    dict(t=(301, 5)),     # budget above T
    dict(n=(0, 50)),      # empty head
])
def test_invalid_problems_are_rejected(bad):
    p, keep = _problem(**bad)
    o = amc.make_options()
    out = ctypes.c_uint64(0)
    st = amc.lib().amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out))
    expect = amc.AMC_ERR_UNSUPPORTED if "d" in bad else amc.AMC_ERR_INVALID_ARG
    assert st == expect


def test_invalid_options_are_rejected():
    p, keep = _problem()
    out = ctypes.c_uint64(0)
    L = amc.lib()
    o = amc.make_options(topk=2)  # plain OMP takes one key per iteration
    assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_INVALID_ARG
    o = amc.make_options(select="batched", topk=32, refit_every=16)  # k*R above 255
    assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_UNSUPPORTED
    o = amc.make_options(nnls_tol=-1.0)
    assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_INVALID_ARG
    for g in (-1, 17):
        o = amc.make_options(head_groups=g)
        assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_INVALID_ARG
    o = amc.make_options(head_groups=8)
    assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_OK
    for g in (9, 16):  # inside the range, not run by this build
        o = amc.make_options(head_groups=g)
        assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_UNSUPPORTED
    for fld, bad in (("exact_refit", 4), ("exact_refit", -1), ("digits_in_panel", 2), ("nnls_polish", 9)):
        o = amc.make_options()
        setattr(o, fld, bad)
        assert L.amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_INVALID_ARG


def test_compact_argument_errors_return_before_any_launch():
    """Null pointers and short workspaces are caught on the host: the call
    returns its status without a GPU (a launch here would fail with AMC_ERR_HIP)."""
    p, keep = _problem()
    o = amc.make_options()
    L = amc.lib()
    fake = ctypes.c_void_p(0x10000)
    ws = amc.workspace_size(p, o)
    # missing output pointer
    st = L.amc_compact(ctypes.byref(p), ctypes.byref(o), fake, fake, fake, None, fake, None, fake, None, None, None,
                       0, fake, ws, None)
    assert st == amc.AMC_ERR_INVALID_ARG
    # workspace too small
    st = L.amc_compact(ctypes.byref(p), ctypes.byref(o), fake, fake, fake, None, fake, fake, fake, None, None, None,
                       0, ctypes.c_void_p(0x100000), ws - 256, None)
    assert st == amc.AMC_ERR_WORKSPACE
    # misaligned workspace
    st = L.amc_compact(ctypes.byref(p), ctypes.byref(o), fake, fake, fake, None, fake, fake, fake, None, None, None,
                       0, ctypes.c_void_p(0x100010), ws, None)
    assert st == amc.AMC_ERR_WORKSPACE
    # trace requested without a buffer
    ot = amc.make_options(trace=True)
    st = L.amc_compact(ctypes.byref(p), ctypes.byref(ot), fake, fake, fake, None, fake, fake, fake, None, None, None,
                       0, ctypes.c_void_p(0x100000), ws, None)
    assert st == amc.AMC_ERR_WORKSPACE


def test_budget_limit_and_phi_budget():
    # budgets above the largest supported budget are reported as unsupported
    p, keep = _problem(T=(20000, 200), t=(16385, 5))
    o = amc.make_options()
    out = ctypes.c_uint64(0)
    assert amc.lib().amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_ERR_UNSUPPORTED
    # a Phi budget below the problem's Phi selects the recompute sweep: no Phi in the workspace
    p, keep = _problem()
    stored = amc.workspace_size(p, amc.make_options())
    o = amc.make_options(phi_budget_bytes=1024)
    assert amc.lib().amc_workspace_size(ctypes.byref(p), ctypes.byref(o), ctypes.byref(out)) == amc.AMC_OK
    assert stored - out.value >= 4 * (100 * 300 + 50 * 200)


def test_nnls_entry_validation():
    L = amc.lib()
    arr = (ctypes.c_int64 * 2)(0, 300)
    fake = ctypes.c_void_p(0x10000)
    assert L.amc_nnls(1, arr, fake, fake, fake, 0, 8, 0, 0.0, None, None, None) == amc.AMC_ERR_UNSUPPORTED
    arr = (ctypes.c_int64 * 2)(0, 0)
    assert L.amc_nnls(1, arr, fake, fake, fake, 0, 8, 0, 0.0, None, None, None) == amc.AMC_ERR_INVALID_ARG
    arr = (ctypes.c_int64 * 2)(0, 10)
    assert L.amc_nnls(1, arr, fake, fake, fake, 0, -1, 0, 0.0, None, None, None) == amc.AMC_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert amc.status_string(s)


def test_greedy_swap_budgets_matches_the_oracle():
    """The library's schedule (host code) equals the oracle's on seeded convex curves."""
    import oracle
    import synth
    import numpy as np
    for seed, H, J in [(540, 288, 40), (541, 8, 12), (542, 33, 5)]:
        L = synth.sensitivity_curves(seed, H, J)
        for units in (H, (H * J) // 3, H * J):
            got = amc.greedy_swap_budgets(L, 16, units * 16)
            want = oracle.greedy_swap_budgets(L, 16, units * 16)
            assert got == (want[0], want[1])
    L = synth.sensitivity_curves(543, 4, 5)
    out = (ctypes.c_int64 * 4)()
    Lc = np.ascontiguousarray(L)
    assert amc.lib().amc_greedy_swap_budgets(4, 5, Lc.ctypes.data_as(ctypes.c_void_p), 16, 17, out, None) \
        == amc.AMC_ERR_INVALID_ARG
    assert amc.lib().amc_greedy_swap_budgets(4, 5, Lc.ctypes.data_as(ctypes.c_void_p), 16, 16 * 21, out, None) \
        == amc.AMC_ERR_INVALID_ARG
