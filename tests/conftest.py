"""Test configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need a real MI355X and the built HIP library; everything
else runs on a CPU-only host (``pytest -m "not gpu"``).
"""
import os
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
