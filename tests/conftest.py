import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    """Build the oracle and the input generator once if they are missing."""
    import oracle
    import synth
    for mod in (oracle, synth):
        if not os.path.exists(mod._LIB_PATH):
            mod.build()
    yield
