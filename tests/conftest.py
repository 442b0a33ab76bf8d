import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case")


def pytest_terminal_summary(terminalreporter):
    """GEMM parity: how many elements of each checked output lay beyond the strict bar
    1e-3 + 1e-2*|exact| (each one shown to be the matrix cores' accumulation, see
    tests/mfma_model.py)."""
    try:
        from tests.mfma_model import StrictBarCounter
    except Exception:
        return
    rows = StrictBarCounter.rows
    if not rows:
        return
    tr = terminalreporter
    tot = sum(r[2] for r in rows)
    bey = sum(r[1] for r in rows)
    tr.section("GEMM parity: elements beyond the strict bar 1e-3 + 1e-2*|exact|")
    tr.write_line(f"{len(rows)} checked outputs, {tot} elements, {bey} beyond the strict bar "
                  "(each within the matrix-core accumulation model)")
    for what, b, n, worst in rows:
        if b:
            tr.write_line(f"  {what}: {b} of {n} (worst excess {worst:.3g})")
