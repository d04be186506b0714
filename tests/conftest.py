"""Shared pytest setup: the `gpu` marker and import paths.

Tests marked `gpu` need an MI355X and the built HIP library; everything else
runs on the CPU (oracle pins, host-side argument checks, symbol exports).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle
