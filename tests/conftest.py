import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (needs an MI355X)")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print relF and max-abs of every bf16-tolerance comparison the run made (the full-size
    workloads compare every element of their outputs)."""
    try:
        from tests._util import PARITY_LOG
    except Exception:  # pragma: no cover
        return
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity against the fp64 oracle (relF / max-abs / max-abs past the storage rounding)")
    for what, rf, ma_raw, ma, n in PARITY_LOG:
        tr.write_line(f"{what:60s} elements {n:>11d}  relF {rf:.3e}  max-abs {ma_raw:.3e}  beyond {ma:.3e}")
