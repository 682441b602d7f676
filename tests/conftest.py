import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path through the C ABI)")
    config.addinivalue_line("markers", "big: full-size workload on the GPU (tens of GB of HBM)")


def _ensure(mod):
    if not os.path.exists(mod.LIB):
        mod.build()


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import _build
    _ensure(_build)
    import oracle
    return oracle


@pytest.fixture(scope="session")
def zero_lib():
    from zero_sharded_mixed_02_amd import _build
    _ensure(_build)
    import zero_sharded_mixed_02_amd as Z
    Z.load()
    return Z


@pytest.fixture(scope="session")
def gpu(zero_lib):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from synth import _build
    _ensure(_build)
    yield torch.device("cuda:0")
    # At the end of the session, hand the memory torch's allocator still holds
    # back to the driver and wait until the memory system has absorbed the
    # release (kernels that stream HBM run a few percent slower for about a
    # second per ~30 GB released), so that whatever runs on the GPU next does
    # not start inside that aftermath.
    import bench
    bench.release(torch)
