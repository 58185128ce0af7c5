import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """Worst err/bound of the GEMM acceptance gate per test (1.0 = at the bound)."""
    from tests._helpers import GATE_MARGINS
    if not GATE_MARGINS:
        return
    worst = {}
    for test, n, ratio, nrm in GATE_MARGINS:
        w = worst.setdefault(test, [0, 0.0, 0.0])
        w[0] += n
        w[1] = max(w[1], ratio)
        w[2] = max(w[2], nrm)
    terminalreporter.write_sep("-", "GEMM gate margins: worst err/bound, normwise error, elements checked")
    for test, (n, ratio, nrm) in sorted(worst.items(), key=lambda kv: -kv[1][1]):
        terminalreporter.write_line(f"{ratio:7.4f}  {nrm:.2e}  {n:>10d}  {test}")
