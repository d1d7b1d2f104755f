import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_sessionfinish(session, exitstatus):
    # GPU parity tests record (case, raw max |d|, excess over the bf16 rounding
    # allowance, mean |d|) through _helpers.assert_parity; with
    # LAZYATTN_PARITY_RECORD=<path> they are written out as a table
    path = os.environ.get("LAZYATTN_PARITY_RECORD")
    if not path:
        return
    try:
        import _helpers
    except ImportError:
        return
    if _helpers.PARITY_RECORDS:
        _helpers.write_parity_records(path)
