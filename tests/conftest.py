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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _hip_library_built():
    """A fresh checkout has no libkda.so: build it once for the host-side tests (hipcc
    cross-compiles gfx950 without a GPU). The binding itself never builds; it raises
    when the library is missing."""
    import gated_delta_rule_98_amd as pkg

    if not os.path.exists(pkg.LIB_PATH):
        from gated_delta_rule_98_amd import build

        build.build()
