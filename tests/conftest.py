import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture
def kas_options():
    """Set library tuning options for one test; every option touched is put
    back to its default afterwards."""
    import sparse_attention_long_anchor_amd as kas
    touched = []

    def setter(option, value):
        touched.append(option)
        kas.set_option(option, value)

    yield setter
    for option in touched:
        kas.set_option(option, -1)
