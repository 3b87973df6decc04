import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle._load()
    return oracle


def log(msg: str) -> None:
    """Progress line that names the case, flushed before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()
