import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """Aggregate of the session's oracle replays: how many heads, how many
    were held to the NNLS minimum value only (non-identifiable beta), the
    largest beta difference and e_out difference among the others, and the
    smallest relative mass residual replayed."""
    mod = sys.modules.get("amc_check")
    reps = getattr(mod, "REPORTS", None) if mod else None
    if not reps:
        return
    gated = [r for r in reps if not r.get("fallback")]
    fb = len(reps) - len(gated)
    bmax = max((r["beta_maxdiff"] for r in gated), default=0.0)
    emax = max(r["e_out_diff"] for r in reps)
    rmin = min(r.get("rel_resid", 1.0) for r in reps)
    tmax = max(r.get("t", 0) for r in reps)
    terminalreporter.write_line(
        f"oracle replays: {len(reps)} heads (largest budget {tmax}), {fb} on the residual gate; "
        f"max beta diff {bmax:.2e} on the others; max e_out diff {emax:.2e}; "
        f"smallest relative residual {rmin:.2e}")
