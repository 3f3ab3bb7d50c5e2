"""Shared pytest configuration: the `gpu` marker, golden-file parsing and library fixtures."""
from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")
    config.addinivalue_line("markers", "slow: full-size workload (still bounded to seconds of oracle time)")


def read_golden(name: str) -> dict[str, list[str]]:
    """Parse a `key: v1 v2 ...` fixture, ignoring `#` comment lines."""
    out: dict[str, list[str]] = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            out[key.strip()] = rest.split()
    return out


def golden_ints(name: str, key: str) -> list[int]:
    return [int(v, 0) for v in read_golden(name)[key]]


def golden_floats(name: str, key: str) -> list[float]:
    return [float(v) for v in read_golden(name)[key]]


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.load()
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0; skips only when torch sees no GPU at all."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import gemm_e2m1_lut_amd as g
    g.load_library()
    return g
