import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: runs the oracle on large inputs (minutes of CPU)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The GPU path: a visible gfx950 device and the built library. Fails
    (does not skip) when either is missing, so a GPU run cannot pass silently."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from point_cloud_neighbor_amd import ops
    ops.device_check()
    return ops
