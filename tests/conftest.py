import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check (needs a GPU)")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    """The oracle and the generator are plain gcc builds; build them if they are missing."""
    import oracle
    import synth

    if not os.path.exists(synth.OBJ) or not os.path.exists(synth.LIB):
        synth.build()
    if not os.path.exists(oracle.LIB):
        oracle.build()
    yield
