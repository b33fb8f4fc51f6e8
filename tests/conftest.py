import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload checks (minutes)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """How many bf16 LayerNorm / log-softmax outputs passed only through the
    fp32 floor of tests/compare.py (more than 1 bf16 ulp from the oracle)."""
    try:
        from tests import compare
    except Exception:
        return
    for op, n in compare.FLOOR_ONLY.items():
        total = compare.FLOOR_CHECKED[op]
        if total:
            terminalreporter.write_line(f"bf16 {op} outputs passing only through the fp32 floor: {n} of {total}")
