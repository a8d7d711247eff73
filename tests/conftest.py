"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else runs
on the CPU.  torch is imported first so that the HIP runtime it ships is the one the
GPU library binds to when it is loaded.
"""
import os
import sys

import pytest
import torch  # noqa: F401  (see module docstring)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle

    return oracle.get()
