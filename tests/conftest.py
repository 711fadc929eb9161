"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; all
other tests run on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; skips when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_sparse_attention_avg_amd as bsa
    bsa.load()          # raises if the shared library is missing
    return bsa
