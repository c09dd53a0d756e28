import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A planted oracle mistake (tests/oracle_mutants.py), applied before any test
# module imports the oracle; set only by test_oracle_mutants.py's subprocesses.
if os.environ.get("BEAM_ORACLE_MUTANT"):
    import oracle_mutants
    oracle_mutants.apply(os.environ["BEAM_ORACLE_MUTANT"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: Beam-shape case that takes tens of seconds")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
