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
def orc():
    import oracle

    return oracle


@pytest.fixture(scope="session")
def moelib():
    """The built HIP library's Python binding (builds it first if it is missing)."""
    from sparsely_gated_mixture_gate_amd import build as _b

    if not os.path.exists(_b.LIB):
        _b.build()
    import sparsely_gated_mixture_gate_amd as m

    m.lib()  # fails here, loudly, if the library cannot be loaded
    return m
