import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    if not os.path.exists(os.path.join(ROOT, "oracle", "libspec_verify_oracle.so")):
        oracle.build(force=True)
    return None  # None selects the default oracle build


def pytest_runtest_logstart(nodeid, location):
    # Name each test on stderr before it runs, so a run that dies on the GPU
    # still shows which case was in flight.
    if "gpu" in nodeid or "smoke" in nodeid:
        sys.__stderr__.write(f"[start] {nodeid}\n")
        sys.__stderr__.flush()
