"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host side only (each -fsanitize= goes to the
host compilation; the GPU code is built as usual), and every host-only ABI test
(tests/test_abi_host.py: config checks, schedule builder and simulator, attention split,
argument errors, the static-workspace size check) runs against that build in a child process
with the ASan runtime preloaded.  Any sanitizer report fails the test: ASan aborts on its first
error and UBSan is built not to recover.  No GPU call is made.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "persistent_moe_decode_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.slow


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None, reason="hipcc or the ASan runtime missing")
def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    from persistent_moe_decode_amd import build
    lib = str(tmp_path / "libmk_asan.so")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + host_san
    cmd = [HIPCC, *flags, "-o", lib, *[os.path.join(CSRC, s) for s in build.SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-3000:]
    # the host code is instrumented (calls into both runtimes)
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), MK_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider"], capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
