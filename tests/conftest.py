"""Shared pytest set-up: repo root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; on a
machine without a GPU they are skipped with that reason.  Everything else runs
on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


_gpu_ok = None


def _have_gpu():
    global _gpu_ok
    if _gpu_ok is None:
        try:
            import torch
            _gpu_ok = bool(torch.cuda.is_available())
        except Exception:  # pragma: no cover - torch missing
            _gpu_ok = False
    return _gpu_ok


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None and not _have_gpu():
        pytest.skip("no GPU visible to torch")
