"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the host sources are rebuilt with the sanitizers and the ABI tests
run against that build in a child process under the clang ASan runtime; any
sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_abi_tests_clean_under_host_sanitizers():
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    from hstu_sequential_transducer_amd import build_asan
    lib = build_asan.build()
    rt = build_asan.runtime()
    if not rt:
        pytest.skip("clang ASan runtime not found")
    env = dict(os.environ, HSTU_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
