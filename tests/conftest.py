import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build()
    return oracle


def pytest_sessionfinish(session, exitstatus):
    """With LA_MARGINS_OUT set, write the worst parity ratio of every checked
    tensor (tests._gpu.MARGINS) to that file as JSON."""
    path = os.environ.get("LA_MARGINS_OUT")
    if not path:
        return
    from tests import _gpu
    import json

    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(_gpu.MARGINS, f, indent=1, sort_keys=True)
