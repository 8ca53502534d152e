"""The host code of the library (problem validation, geometry, CSR layout, stream-state checks, the
backward's workspace layout, every rejection path) run under AddressSanitizer and
UndefinedBehaviorSanitizer: a build whose host pass carries both sanitizers loads into a Python with
the ASan runtime preloaded, and the whole host ABI test module runs against it. Any sanitizer report
aborts the child process and fails this test. CPU only: no entry point launches a kernel here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib():
    from block_sparse_causal_lcsa_amd import build
    return build.build_host_sanitized(), build.sanitizer_runtime()


def test_sanitized_library_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE, text=True,
                          check=True).stdout
    assert "__asan_report_load" in syms or "__asan_load" in syms
    assert "__ubsan_handle_" in syms


def test_host_abi_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    assert os.path.exists(rt), rt
    env = dict(os.environ, LCSA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
