import os
import sys

import pytest

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
for p in (_ROOT, _HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (seconds to a minute)")


@pytest.fixture(scope="session")
def lib():
    """The HIP library, loaded once; GPU tests fail loudly when it is missing."""
    import paged_gqa_decode_step_amd as sa
    sa.load()
    return sa
