import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmhc.so")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionfinish(session, exitstatus):
    mod = sys.modules.get("mhc_testlib")
    if mod is not None:
        mod.write_stats()
