"""Test configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an MI355X (gfx950) and the built ``libkvattn.so``; everything else runs
on the CPU. A GPU test never skips silently for a missing device or library: it fails.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
