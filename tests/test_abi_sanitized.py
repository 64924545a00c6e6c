"""The C ABI's host code (argument validation, aliasing checks, launch plans, workspace sizes, status
strings) under AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt with both on its host
compilation (device code unchanged) and tests/test_abi.py runs against it in a child process that preloads
the ASan runtime.  Any sanitizer report aborts the child and fails this test.  No GPU is needed: every ABI
test stops at host validation."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from selective_state_space_05_amd import build as BLD

ROOT = Path(__file__).resolve().parents[1]


@pytest.mark.slow
def test_abi_suite_under_asan_and_ubsan(tmp_path):
    lib = BLD.build_sanitized(tmp_path / "libsamba_scan_sanitized.so")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": str(BLD.asan_runtime()),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "SAMBA_ABI_TEST_LIBRARY": str(lib),
    })
    res = subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / "test_abi.py"), "-q", "-x",
                          "-p", "no:cacheprovider", "-m", "not gpu"],
                         cwd=str(ROOT), env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, "ABI suite under ASan/UBSan failed (exit %d):\n%s" % (res.returncode, tail)
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in res.stdout
