import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def _ensure_built():
    """Build the oracle and the product library when either is missing or
    was built from other sources than the ones in the tree (each build
    records a hash of its sources beside the library); a current build is
    used as is."""
    from oracle import build as oracle_build
    from rotary_position_embedding_amd import build as product_build
    if not oracle_build.is_current() or not product_build.is_current():
        import __graft_entry__ as ge
        ge.build()


_ensure_built()
