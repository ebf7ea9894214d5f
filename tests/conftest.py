import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")
    # a planted mistake in the oracle (tests/test_oracle_mutations.py runs the pins against
    # each one in a child process; CPU only)
    mutant = os.environ.get("CSA2_ORACLE_MUTANT")
    if mutant:
        from tests import _mutants

        _mutants.apply(mutant)


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a CPU-only host they are skipped
    # with a reason rather than failing (the CPU suite runs with -m "not gpu").
    try:
        import torch

        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
