import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (seconds to a minute)")


def pytest_terminal_summary(terminalreporter):
    """Positions where a GPU result and the oracle's differ only inside the
    fp32 rounding allowance (tests/parity.py), listed per test."""
    try:
        from parity import RELAXED
    except ImportError:
        return
    if not RELAXED:
        return
    terminalreporter.section("positions relaxed within the fp32 bound")
    per = {}
    for test, m, i, g, o in RELAXED:
        per.setdefault(test, []).append(f"row {m} pos {i}: gpu {g} oracle {o}")
    for test, items in per.items():
        terminalreporter.write_line(f"{test}: {len(items)}")
        for it in items[:10]:
            terminalreporter.write_line(f"    {it}")
