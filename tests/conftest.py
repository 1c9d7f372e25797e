import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # load what is built; build only when nothing is (hipcc cross-compiles without a GPU)
    import fine_grained_block_amd as fgb
    if not os.path.exists(fgb.LIB_PATH):
        from fine_grained_block_amd import build
        build.build_library()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()            # builds the library when it is missing or older than its source
    return oracle
