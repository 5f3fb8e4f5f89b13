import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    from tests import parity
    hits = parity.VACUOUS_HITS
    terminalreporter.write_line(
        f"parity: {len(hits)} compared slice(s) passed through the vacuity rule "
        f"(every |reference| <= {parity.VACUOUS:g})")
    for ref_inf, rel, shape in hits[:20]:
        terminalreporter.write_line(f"  max|ref|={ref_inf:.3e} rel_l2={rel:.3e} shape={shape}")
