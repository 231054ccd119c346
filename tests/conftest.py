import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    out = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def golden_constants():
    vals = {}
    for line in read_golden("flint_constants.txt"):
        k, v = [p.strip() for p in line.split("=")]
        vals[k] = float(v)
    return vals
