import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture into a list of record dicts."""
    path = os.path.join(ROOT, "tests", "golden", name)
    recs, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "name":
                cur = {"name": rest}
                recs.append(cur)
            elif cur is not None:
                cur[key] = rest
            else:
                recs.append({key: rest})
    return recs


def expand_list(s, cast=float):
    out = []
    for tok in s.split():
        if "*" in tok:
            v, n = tok.split("*")
            out += [cast(v)] * int(n)
        else:
            out.append(cast(tok))
    return out
