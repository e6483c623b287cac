import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size CPU work (several seconds)")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    # the oracle and the input generator are plain C; build them once if missing
    import oracle
    import synth
    synth.lib()
    oracle.lib()
    yield
