import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU sweep")


@pytest.fixture(scope="session")
def markstein_lib():
    """Build the test-side check of the NVFP4 coder's division (tests/helpers/markstein_div.c)."""
    import ctypes
    src = os.path.join(ROOT, "tests", "helpers", "markstein_div.c")
    out = os.path.join(tempfile.mkdtemp(prefix="fgq_helpers_"), "libmarkstein.so")
    subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", src, "-o", out, "-lm"])
    lib = ctypes.CDLL(out)
    lib.markstein_sweep.restype = ctypes.c_uint64
    lib.markstein_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.POINTER(ctypes.c_uint64),
                                    ctypes.POINTER(ctypes.c_uint64),
                                    ctypes.POINTER(ctypes.c_uint64)]
    return lib


@pytest.fixture(scope="session")
def helper_lib():
    """Build the test-side helper C code (independent of the oracle) into a temp dir."""
    import ctypes
    src = os.path.join(ROOT, "tests", "helpers", "e4m3_bitenc.c")
    out = os.path.join(tempfile.mkdtemp(prefix="fgq_helpers_"), "libhelpers.so")
    subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", src, "-o", out])
    lib = ctypes.CDLL(out)
    lib.helper_bitenc.restype = ctypes.c_uint8
    lib.helper_bitenc.argtypes = [ctypes.c_float]
    lib.helper_sweep.restype = ctypes.c_uint64
    lib.helper_sweep.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.POINTER(ctypes.c_uint64)]
    return lib
