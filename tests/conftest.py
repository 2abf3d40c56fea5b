"""pytest configuration: the ``gpu`` marker and shared helpers.

Tests marked ``gpu`` need an MI355X (gfx950) and the built ``libfa.so``; the
rest run on any CPU host.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A gpu test on a host without a GPU is an error in test selection, not a
    # skip: the round-end GPU run must never pass by skipping. Only when the
    # selection explicitly excludes gpu tests are they deselected by -m.
    pass
