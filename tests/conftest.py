import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library on cuda:0)")


def read_golden(name):
    """Parse a golden fixture: '# ...' comments; 'key: v1 v2 ...' lines; a 'key:' line with
    no values opens a block whose following bare rows are collected under that key; bare
    rows outside a block go under '_rows'."""
    out, block = {}, "_rows"
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                k, v = line.split(":", 1)
                k, v = k.strip(), v.split()
                if v:
                    out[k] = v
                    block = "_rows"
                else:
                    out[k] = []
                    block = k
            else:
                out.setdefault(block, []).append(line.split())
    return out
