import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def fdec():
    """The HIP library's Python binding, built in-tree first if nothing is built."""
    import decode_attention_fdec_amd as f

    if not os.path.exists(f.LIB_PATH):
        from decode_attention_fdec_amd import build

        build.build()
    f.load_library()
    return f
