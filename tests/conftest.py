import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def load_golden(name):
    """Parse a tests/golden fixture: '[section]' headers, 'key: values' lines,
    and 'mask:' followed by rows of 0/1."""
    path = os.path.join(ROOT, "tests", "golden", name)
    sections, cur, in_mask = {}, None, False
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                in_mask = False
                continue
            if line.startswith("["):
                cur = sections.setdefault(line.strip("[]"), {})
                in_mask = False
                continue
            if in_mask and set(line) <= {"0", "1"}:
                cur["mask"].append([int(c) for c in line])
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            in_mask = key == "mask"
            if in_mask:
                cur["mask"] = []
            elif key == "nodes":
                cur[key] = val.split()
            else:
                cur[key] = [int(x) for x in val.split()]
    return sections


@pytest.fixture
def golden():
    return load_golden
