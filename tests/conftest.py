import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


def read_golden(name: str):
    """Non-comment lines of a golden fixture, split on whitespace."""
    out = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            out.append(line.split())
    return out


def golden_bytes(rows, key: str) -> bytes:
    for r in rows:
        if r[0] == key + ":":
            return bytes(int(t, 16) for t in r[1:])
    raise KeyError(key)
