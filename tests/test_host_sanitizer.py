"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second copy of the library is built with the host side instrumented (the
device code is compiled as for the product library) and loaded into a child
process that preloads the AddressSanitizer runtime.  There, the driver
(tests/sanitizer_driver.py) runs every host path that needs no GPU: the
block-32 scale packer on success and on each refusal, the argument checks of
every entry point, and the plan, workspace and limits queries over a sweep of
shapes.  An out-of-bounds access, use-after-free, signed overflow, bad shift
or misaligned load in that code aborts the child with a report, which fails
the test.  No GPU: nothing here launches a kernel.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from blockwise_scaled_fp8_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(600)
def test_host_paths_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("AddressSanitizer runtime not found under /opt/rocm/llvm")
    lib = build.build_host_sanitized(str(tmp_path / "libbfp8_hostsan.so"))
    env = dict(os.environ)
    # every allocation through malloc, so the runtime's redzones surround it
    env.update(LD_PRELOAD=runtime, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, os.path.join(HERE, "sanitizer_driver.py"), lib],
                       env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "host paths ok" in p.stdout, p.stdout[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer"):
        assert marker not in p.stdout, p.stdout[-4000:]
