import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_libs():
    """Host-side libraries (oracle, generator) are tiny: build them if absent."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(synth.LIB_PATH):
        synth.build(gpu=False)
