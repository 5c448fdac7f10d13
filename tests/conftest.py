import ast
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libspattn.so")


def load_golden(name: str) -> dict:
    """Parse a fixture of ``key = <python literal>`` statements (comments allowed)."""
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        tree = ast.parse(f.read())
    out = {}
    for node in tree.body:
        assert isinstance(node, ast.Assign) and len(node.targets) == 1
        out[node.targets[0].id] = ast.literal_eval(node.value)
    return out


@pytest.fixture
def golden():
    return load_golden
