import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them instead of failing when selected.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Report the near-tie tally of the GPU parity tests (sampled tokens and accept
    decisions compared with the oracle; flagged = inside the near-tie threshold; excused =
    flagged and decided otherwise by the GPU)."""
    mod = sys.modules.get("gpu_round")
    if mod is None:
        return
    t = mod.TALLY
    if not (t["samples"] or t["accept_tests"]):
        return
    rate = t["flagged"] / t["samples"] if t["samples"] else 0.0
    terminalreporter.write_line(
        f"NEAR-TIE TALLY: {t['samples']} sampled tokens compared, {t['flagged']} flagged "
        f"(oracle top-2 gap < 1e-4; rate {rate:.2e}), {t['excused']} excused mismatches; "
        f"{t['accept_tests']} accept decisions, {t['accept_flagged']} flagged (margin < 1e-5), "
        f"{t['accept_excused']} excused")
