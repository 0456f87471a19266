import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available() -> bool:
    try:
        import torch
    except Exception:  # pragma: no cover
        return False
    return bool(torch.cuda.is_available())


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build()
    return oracle


_WORKLOADS = {}


@pytest.fixture(scope="session")
def workload_cache():
    """Named workloads drawn once per session (config 5 holds about 1.4 GB of pools)."""
    from synth import make_workload

    def get(config: int):
        if config not in _WORKLOADS:
            _WORKLOADS[config] = make_workload(config)
        return _WORKLOADS[config]

    return get
