"""Shared pytest setup: the `gpu` marker, import paths, and the GPU-availability gate."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def pytest_collection_modifyitems(config, items):
    gpu_tests = [it for it in items if "gpu" in it.keywords]
    if not gpu_tests:
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in gpu_tests:
        it.add_marker(skip)
