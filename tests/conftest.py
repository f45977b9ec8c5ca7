"""Shared test setup: import paths and the ``gpu`` marker.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; all
other tests run on the CPU.
"""
import os
import sys

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
