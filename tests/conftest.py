import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_report_header(config):
    # which build of the library the binding loads (FA355_LIBRARY selects another one)
    from exact_io_aware_65_amd._binding import LIBRARY
    return f"libfa355 under test: {LIBRARY}"
