import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error figure of every parity check of the session, so that
    the session's tail carries them."""
    try:
        from tests.tolerance import RECORDS
    except Exception:  # pragma: no cover
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("parity error figures (max abs, max / RMS(ref), RMS err / RMS(ref), bar)")
    for test, name, f in RECORDS:
        if "max_over_rms" in f:
            bar = f"{f['rel']:.0e}*RMS" + (f" + {f['store_term'] * 256:.0f}*2^-8|x|" if f["store_term"] else "")
            tr.write_line(f"{test} {name}: max {f['max_abs']:.3e} = {f['max_over_rms']:.5f} RMS, "
                          f"rms err {f['rel_rms']:.5f}; bar {bar}")
        else:
            tr.write_line(f"{test} {name}: max abs {f['max_abs']:.3e}; bar {f['bar']:.0e}")
