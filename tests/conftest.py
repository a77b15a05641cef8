import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None:
        # Name the case before any GPU work so a crash log says where it was.
        print(f"\n[gpu-case] {item.nodeid}", flush=True)


@pytest.fixture(scope="session")
def golden():
    import json

    with open(os.path.join(ROOT, "tests", "golden", "worked_tokens.json")) as f:
        return json.load(f)
