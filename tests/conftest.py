import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The parity margin of every GPU comparison, per test family."""
    mod = sys.modules.get("tests.gpu_util")
    if mod is None or not mod.RECORDS:
        return
    terminalreporter.section("parity margins (max|err| <= 1e-2 bound, cos >= 0.99998)")
    for line in mod.summary_lines():
        terminalreporter.write_line(line)
