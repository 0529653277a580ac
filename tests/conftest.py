import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    from tests import parity_log
    lines = parity_log.lines()
    if lines:
        terminalreporter.write_sep("-", "whole-output parity at full size")
        for line in lines:
            terminalreporter.write_line(line)
