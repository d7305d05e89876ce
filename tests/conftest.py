import json
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def parse_num(x):
    """Golden numbers may be written as 'lnK' (natural log of K)."""
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        return float(x)
    return float(x)
