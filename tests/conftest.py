import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# The sanitizer build of the library's host-only checks (tests/test_host_sanitizers.py runs the
# host ABI tests against it in a child process): the binding's functions then call it.
_HOST_CHECK_LIB = os.environ.get("MPGEMM_HOST_CHECK_LIB")
if _HOST_CHECK_LIB:
    import ctypes

    import mixed_precision_dense_amd as _mp
    _mp._lib = _mp.declare(ctypes.CDLL(_HOST_CHECK_LIB))
