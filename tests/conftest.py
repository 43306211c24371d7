"""Shared pytest setup: the ``gpu`` marker, golden-fixture reader, oracle build."""
from __future__ import annotations

import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) device; runs the HIP path")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if any("gpu" in item.keywords for item in items) and not _gpu_available():
        skip = pytest.mark.skip(reason="no GPU visible")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)


def read_golden(name: str) -> dict[str, list[str]]:
    """Parse a ``key: values`` fixture (``#`` lines are citations/comments)."""
    out: dict[str, list[str]] = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(":")
        out[key.strip()] = rest.split()
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden
