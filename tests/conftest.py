"""Shared test configuration.

Marker ``gpu``: needs a gfx950 GPU and the built HIP library; everything else
runs on the CPU (oracle pins, host-side argument validation, symbol exports).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def ora():
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def syn():
    import synth

    synth._L()
    return synth
