import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter):
    """Largest GPU-vs-oracle errors of the run, per dtype, beside the bounds."""
    mod = sys.modules.get("parity_util")
    if mod is None or not (mod.MAX_SEEN["o"] or mod.MAX_SEEN["lse"]):
        return
    tr = terminalreporter
    tr.write_sep("-", "largest errors against the oracle")
    for kind, bounds in (("o", mod.TOL), ("lse", mod.LSE_TOL)):
        for dt, err in sorted(mod.MAX_SEEN[kind].items()):
            tr.write_line("%-3s %-4s max|err| = %.3g  (bound %.0e)" % (kind, dt, err, bounds[dt]))
