import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.Oracle()


_cache = {}


@pytest.fixture(scope="session")
def workload_inputs():
    """Generated inputs, cached per (name, with_x) for the session."""
    from combine_ep_get_02_amd import inputs

    def get(name, with_x=True):
        key = (name, with_x)
        if key not in _cache:
            _cache[key] = inputs.generate(name, with_x=with_x)
        return _cache[key]

    return get
