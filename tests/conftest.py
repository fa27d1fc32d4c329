"""Shared pytest configuration.

Markers:
  gpu  -- needs an MI355X (gfx950) and the built HIP library; these are the
          parity tests proper and call the library through its C ABI.
  slow -- CPU tests that take more than a few seconds (exhaustive sweeps).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test (exhaustive sweep)")


def load_golden(name):
    """Read a tests/golden/*.txt fixture: '#' comments, 'key = value' lines."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out
