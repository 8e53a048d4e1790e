"""Shared pytest setup: the repository root on sys.path and the gpu marker."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _fmt(x):
    return "%.2e" % x if isinstance(x, float) else str(x)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the figures of every parity check that ran (parity.FIGURES):
    forward: gate distance to the bf16 rounding cell (o_max), literal max
    |O - O_exact| (o_max_fp64), max against bf16(O_exact), mean |dO| and
    max |dLSE|; all-outputs checks against the fp32 reference: the same
    cell distance over every output; gradients: max error, use of the
    elementwise bound and relative RMS error."""
    parity = sys.modules.get("parity")
    if parity is None or not getattr(parity, "FIGURES", None):
        return
    tr = terminalreporter
    tr.section("parity figures (%d checks)" % len(parity.FIGURES))
    keys = {
        "forward": ("o_max", "o_max_fp64", "o_max_vs_bf16_exact", "o_mean", "lse_max"),
        "all-outputs": ("o_max", "o_max_vs_bf16_ref", "o_mean", "lse_max", "outputs"),
        "gradient": ("max_err", "bound_use", "rel_rms"),
    }
    for test, what, kind, st in parity.FIGURES:
        name = test.split("::", 1)[-1]
        figs = " ".join("%s=%s" % (k, _fmt(st[k])) for k in keys.get(kind, ()) if k in st)
        tr.write_line("%-11s %s | %s | %s" % (kind, name, what, figs))
