"""Shared pytest set-up: markers and session fixtures.

``-m "not gpu"`` runs on any host: the oracle against its pins, host-side
logic and the C-ABI library's symbol table and argument checks.  ``-m gpu``
tests need an MI355X and call the HIP library through its C ABI.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: larger sizes; still minutes at most")


@pytest.fixture(scope="session")
def oracle_lib():
    # tests/test_sanitizers.py runs the oracle's pins again on a copy built
    # with AddressSanitizer and UndefinedBehaviorSanitizer, named here.
    import oracle
    return oracle.load(os.environ.get("MHC_TEST_ORACLE_LIB") or None)
