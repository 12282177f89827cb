"""Shared pytest set-up: the ``gpu`` marker and import paths.

Tests marked ``gpu`` call the HIP library through its C ABI and need an MI355X;
everything else (the oracle's pins, input generation, host-side argument
checks, symbol export) runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
