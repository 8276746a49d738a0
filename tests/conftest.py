import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Build the HIP library (cross-compiles for gfx950, no GPU needed) and the oracle if absent."""
    from persistent_decode_megakernel_02_amd import build as mkbuild
    if not os.path.exists(mkbuild.LIB):
        mkbuild.build()
    from oracle import build as obuild
    obuild.ensure_built()
    yield
