"""The host-side code under AddressSanitizer + UndefinedBehaviorSanitizer:
packing and argument checks of the C ABI, the host leg, the residency
policy, the oracle and the input generator (tests/sanitize/driver.cpp,
built by tests/sanitize/build.py).  CPU only."""
import os
import subprocess

import pytest

from tests.sanitize import build as SB


@pytest.fixture(scope="module")
def driver():
    return SB.build()


def test_host_code_is_clean_under_asan_and_ubsan(driver):
    supp = os.path.join(os.path.dirname(SB.__file__), "lsan.supp")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "all passed" in r.stdout
