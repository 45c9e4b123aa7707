"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The sources are rebuilt with -fsanitize=address,undefined on the host pass
only (the device code is unchanged), and the host-side ABI suite
(tests/test_abi_host.py: plan, argument checks, workspace sizes, status
strings) runs against that build in a child process that preloads clang's
shared ASan runtime.  Any report (out-of-bounds access, use after free,
signed overflow, invalid enum or shift, misaligned load) ends the child with
a non-zero status.  No GPU is used.
"""
import os
import subprocess
import sys

import pytest

from block_wise_mixed_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("clang's shared ASan runtime is not installed")
    out = str(tmp_path_factory.mktemp("asan") / "libmsq_asan.so")
    build.build_host_sanitized(out)
    return out, rt


def test_library_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                          text=True, check=True).stdout
    assert "__asan_report_load" in syms
    assert "__ubsan_handle_" in syms


@pytest.mark.timeout(600)
def test_host_abi_suite_clean_under_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        # the HIP runtime keeps process-lifetime allocations; leaks are not checked
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONMALLOC": "malloc",
        "MSQ_LIBRARY": lib,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    log = r.stdout + r.stderr
    assert "Sanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in r.stdout
