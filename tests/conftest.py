import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: `key = value` lines, '#' comments."""
    path = os.path.join(HERE, "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(x) if any(c in x for c in ".e") else int(x) for x in v.split()]
            out[k] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden


@pytest.fixture(scope="session")
def libmqa_path():
    """Path of the built libmqa.so, compiling it first when it is missing."""
    from query_decode_attention_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    return B.LIB
