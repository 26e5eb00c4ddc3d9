"""Shared pytest setup: markers, import path, and building what is missing.

``gpu`` marks tests that need an MI355X (gfx950).  Everything else runs on a
CPU-only host.  Nothing here is rebuilt if the built libraries exist; after a
source change run ``__graft_entry__.build()``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    import __graft_entry__ as ge
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        ge.build_oracle()


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN
