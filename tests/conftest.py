import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    try:
        from fgtest import PARITY
    except Exception:   # the GPU helpers are not importable without torch
        return
    if PARITY:
        terminalreporter.write_sep("-", "whole-output parity against the oracle")
        for line in PARITY:
            terminalreporter.write_line(line)
