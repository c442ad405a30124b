import ctypes
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_crashnote = None


def _load_crashnote():
    """Build and install the native fatal-signal reporter (tests/crashnote.c); None if gcc is
    missing. It must be installed before pytest enables faulthandler, which then chains to it."""
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "crashnote.c")
    try:
        out = os.path.join(tempfile.mkdtemp(prefix="crashnote_"), "libcrashnote.so")
        subprocess.run(["gcc", "-O1", "-shared", "-fPIC", src, "-o", out], check=True, capture_output=True,
                       timeout=60)
        lib = ctypes.CDLL(out)
        lib.crashnote_set.argtypes = [ctypes.c_char_p]
        if lib.crashnote_install() != 0:
            return None
        return lib
    except Exception:
        return None


@pytest.hookimpl(tryfirst=True)
def pytest_configure(config):
    global _crashnote
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    _crashnote = _load_crashnote()


def pytest_runtest_logstart(nodeid, location):
    # the test id goes out unbuffered before the test runs, so that a record of a crash names it
    sys.__stderr__.write(f"[test start] {nodeid}\n")
    sys.__stderr__.flush()
    if _crashnote is not None:
        _crashnote.crashnote_set(nodeid.encode())
