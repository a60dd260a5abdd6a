"""Shared pytest configuration.

Markers:
  gpu  -- needs an MI355X (gfx950) and the built HIP library; run with ``-m gpu``.
Tests without the marker run on any CPU host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run where no GPU is visible; say so instead of failing obscurely.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
