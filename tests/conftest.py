import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the device)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """Worst error/bound of the parity checks that ran (GPU runs), so that the end
    of the log shows how close each workload came to its bound."""
    mod = sys.modules.get("parity_util")
    res = getattr(mod, "RESULTS", None)
    if not res:
        return
    tr = terminalreporter
    tr.section("parity: max error / bound (1.0 = at the bound)")
    key = ("_bf16", "_f32", "shared", "split", "whole", "phase")
    shown = [r for r in res if any(k in r[0] for k in key)]
    for what, err, ratio in shown[-40:]:
        tr.write_line(f"{ratio:7.3f}  max err {err:.3e}  {what}")
    worst = max(res, key=lambda r: r[2])
    tr.write_line(f"worst of {len(res)} checks: {worst[2]:.3f} ({worst[0]})")
