"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the library's argument checks, error strings and
status paths are rebuilt with both sanitizers (device code unchanged) and
the whole ABI test module runs against that build in a child process, with
the sanitizer runtime preloaded and any report fatal.  Runs on the CPU."""

import os
import subprocess
import sys

import pytest

from exact_tiled_self_amd.build import asan_runtime, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    return build(out=str(tmp_path_factory.mktemp("san") / "libattn_san.so"), sanitize=True)


def test_abi_tests_pass_under_asan_and_ubsan(san_lib):
    env = dict(os.environ)
    env.update({
        "ATTN_LIBRARY": san_lib,
        "LD_PRELOAD": asan_runtime(),
        # the interpreter itself is not instrumented: its allocations at exit
        # are not the library's leaks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    proc = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                           "-q", "-x", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)
    report = proc.stdout[-3000:] + proc.stderr[-3000:]
    assert proc.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert " passed" in proc.stdout
