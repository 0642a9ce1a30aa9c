"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built ``libmeswish.so``;
everything else runs on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP GPU (MI355X) and libmeswish.so")


@pytest.fixture(scope="session")
def oracle():
    from oracle import Oracle
    return Oracle()
