import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def read_golden(name):
    """key = value lines (repeated keys collect into a list); '#' lines are comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            if k in out:
                if not isinstance(out[k], list) or k not in ("request", "expect"):
                    out[k] = [out[k]] if not isinstance(out[k], list) else out[k]
                out[k].append(v)
            else:
                out[k] = [v] if k in ("request", "expect") else v
    return out
