import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run last within a session so CPU failures surface first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle
