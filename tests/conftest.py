import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Report the secondary attention error measures of the GPU parity tests
    (the bar itself is asserted test by test)."""
    mod = sys.modules.get("tests.gpu_harness")
    if mod is None or not any(mod.ATTN_STATS.values()):
        return
    st = mod.ATTN_STATS
    terminalreporter.write_line(
        f"attention error vs the oracle, worst over this run: {st['block']:.3e} per (layer, request) block, "
        f"{st['per_head']:.3e} per head (both bounded by 2e-3), {st['elementwise_floor']:.3e} elementwise with a "
        f"1e-3 max|ref| floor (reported only)")
