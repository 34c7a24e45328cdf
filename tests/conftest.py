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
    """Build only what is missing; a built tree is used as is."""
    from oracle import LIB_PATH as ORACLE_LIB
    product_lib = os.path.join(ROOT, "rotary_position_embedding_amd", "librope_mi355x.so")
    if not os.path.exists(ORACLE_LIB) or not os.path.exists(product_lib):
        import __graft_entry__ as ge
        ge.build()


_ensure_built()
