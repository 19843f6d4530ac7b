import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_cpu_libs():
    """The oracle and the input generators are plain gcc builds, and the HIP
    library cross-compiles with hipcc without a GPU; each is built only when
    nothing is built yet (after a source change, rebuild with
    __graft_entry__.build())."""
    from oracle import build as ob
    from datagen import build as db
    if not os.path.exists(ob.LIB):
        ob.build()
    if not os.path.exists(db.LIB):
        db.build()
    from bf16_wire_all_amd import build as xb
    if not os.path.exists(xb.LIB):
        xb.build()


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
