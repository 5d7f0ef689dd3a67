"""Shared pytest set-up: the repository root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` need a real MI355X (gfx950) and call the HIP library;
everything else runs on a host without a GPU.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
