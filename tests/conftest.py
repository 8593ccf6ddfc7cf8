"""Shared pytest configuration: the ``gpu`` marker and golden-file reader."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def read_golden(name):
    """Parse a golden fixture: ``key: value`` lines, ``#`` comments, and a
    ``grid:`` key followed by rows of whitespace-separated cells."""
    out = {}
    grid = None
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for raw in f:
            line = raw.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            if grid is not None and ":" not in line:
                grid.append(line.split())
                continue
            key, _, val = line.partition(":")
            key = key.strip()
            val = val.strip()
            if key == "grid":
                grid = []
                out["grid"] = grid
                continue
            grid = None
            out[key] = val
    return out


@pytest.fixture
def golden():
    return read_golden
