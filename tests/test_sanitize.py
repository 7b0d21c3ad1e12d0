"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code
(CPU only): the oracle's C source (tests/sanitize/oracle_driver.c) and the
C ABI's validation and launch planning in api.hip with the kernel launchers
stubbed (tests/sanitize/api_driver.hip).  Each driver exits non-zero on a
failed check or on any sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-o", exe, os.path.join(HERE, "oracle_driver.c"), "-lm"])
    assert "oracle driver ok" in _run(exe)


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_api_host_paths_under_asan_ubsan(tmp_path):
    obj, exe = str(tmp_path / "api_driver.o"), str(tmp_path / "api_driver")
    # the sanitizers instrument the host pass only (the device pass has no
    # kernels here); the link adds their runtimes
    subprocess.check_call([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "quantized_kv_attention_amd", "csrc"),
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=all",
                           "-c", os.path.join(HERE, "api_driver.hip"), "-o", obj],
                          stderr=subprocess.DEVNULL)
    subprocess.check_call([CLANG, "-fsanitize=address,undefined", obj, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
                           "-Wl,-rpath,/opt/rocm/lib"])
    assert "api driver ok" in _run(exe)
