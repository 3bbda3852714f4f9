import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity margins of the layer comparisons (max |y - oracle| / RMS against
    the tolerance of the GEMM path the library took), printed also under -q."""
    h = sys.modules.get("tests._harness")
    margins = getattr(h, "MARGINS", None) if h else None
    if not margins:
        return
    names = {1: "few routes per expert (exact integer operands)",
             2: "many routes per expert (fp16-rounded weights)"}
    tr = terminalreporter
    tr.write_sep("-", "layer parity margins: max|y - oracle| / RMS(oracle)")
    for path in sorted({m[1] for m in margins}):
        ms = [m for m in margins if m[1] == path]
        worst = max(ms, key=lambda m: m[2])
        tr.write_line(f"path {path}, {names.get(path, '?')}: {len(ms)} cases, max {worst[2]:.2e} "
                      f"against tolerance {worst[3]:.0e} ({worst[0]})")
    for case, path, err, tol in margins:
        tr.write_line(f"  {err:.2e} / {tol:.0e}  path {path}  {case}")
