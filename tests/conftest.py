import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the margin of every parity gate this run evaluated (also under -q)."""
    helpers = sys.modules.get("tests.gpu_helpers")
    records = getattr(helpers, "GATE_RECORDS", None) if helpers else None
    if not records:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity gate margins (bar: max_abs <= 1e-2, frac_2ulp >= 0.999, lse <= 1e-3)")
    tr.write_line(f"{'case':<44} {'elements':>11} {'max_abs':>10} {'frac_2ulp':>10} {'lse_max_abs':>11}")
    for label, st in records:
        tr.write_line(f"{label[:44]:<44} {st['elements']:>11d} {st['max_abs']:>10.3e} "
                      f"{st['frac_2ulp']:>10.6f} {st['lse_max_abs']:>11.3e}")
