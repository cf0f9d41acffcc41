import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running statistical test")


# Full-size workloads, generated once per session (tens of seconds each on
# the host) and shared by the parity and statistics tests.  Tests must not
# modify them.


@pytest.fixture(scope="session")
def controlled_full():
    import workloads as W
    print("generating controlled-acceptance B=512 k=8 V=128256 f32 probs", flush=True)
    return W.controlled_acceptance()


@pytest.fixture(scope="session")
def llama3_full():
    import workloads as W
    print("generating sampling chain B=64 k=8 V=128256 bf16", flush=True)
    return W.sample_chain_llama3()
