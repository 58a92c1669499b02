"""The host side of the C ABI -- argument validation, layout and workspace
sizing (api.hip) -- built with AddressSanitizer and UndefinedBehaviorSanitizer
(libwildcat_hostsan.so, made by the build step): test_abi.py runs against
that build in a child process with the sanitizer runtime preloaded, and must
pass with no sanitizer report.  No GPU is needed (no compute calls)."""
import os
import subprocess
import sys

import pytest

from nystr_rpcholesky_coreset_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_tests_clean_under_host_sanitizers():
    if not os.path.exists(B.HOSTSAN_LIB):
        pytest.skip("libwildcat_hostsan.so not built")
    if B.asan_runtime() is None:
        pytest.skip("no AddressSanitizer runtime found")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=B.hostsan_env(), capture_output=True, text=True, timeout=600)
    out = p.stdout + p.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in out
