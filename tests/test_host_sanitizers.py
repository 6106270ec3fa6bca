"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The boundary's host side (argument validation, size arithmetic, workspace
carving, kernel planning and dispatch) is compiled with ASan and UBSan (host
pass only: device code is unchanged) into a separate library, and the CPU
tests of the C ABI and of the dispatcher run against it in
a child process with the sanitizer runtime preloaded.  Any report (an
out-of-bounds access, a use after free, signed overflow, a misaligned or null
dereference, a bad shift) aborts the child, so the test fails with the report
in its output.  Nothing here touches a GPU.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ("-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=undefined "
             "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()
TESTS = ["tests/test_abi.py", "tests/test_dispatch.py"]

PLUGIN = '''
import os


def pytest_configure(config):
    from depth_wise_attention_amd import binding
    binding.LIB_PATH = os.environ["ATTNRES_SANITIZED_LIB"]
'''


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if _asan_runtime() is None or shutil.which("nm") is None:
        pytest.skip("no clang ASan runtime or nm on this host")
    from depth_wise_attention_amd import build

    out = str(tmp_path_factory.mktemp("san") / "libattnres_sanitized.so")
    build.build(out=out, defines=SAN_FLAGS)
    return out


def test_library_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms, "the host code carries no ASan checks"
    assert "__ubsan_handle_" in syms, "the host code carries no UBSan checks"


def test_boundary_tests_pass_under_sanitizers(sanitized_lib, tmp_path):
    (tmp_path / "attnres_sanitized_plugin.py").write_text(PLUGIN)
    env = dict(os.environ)
    env.update({
        "ATTNRES_SANITIZED_LIB": sanitized_lib,
        "PYTHONPATH": os.pathsep.join([str(tmp_path), ROOT, env.get("PYTHONPATH", "")]),
        "LD_PRELOAD": _asan_runtime(),
        # Python and the HIP runtime keep allocations alive until exit by design.
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-p", "attnres_sanitized_plugin", "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", *TESTS]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = p.stdout + p.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert p.returncode == 0, out[-6000:]
    assert " passed" in out and "failed" not in out, out[-3000:]
