"""The C-ABI host layer (argument checks, layout arithmetic) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

zha_api.cpp is compiled with the host sanitizers (device code untouched) and
linked with host-only launcher stubs into a separate library; the CPU ABI
tests (tests/test_abi.py) then run against it in a child process with the
sanitizer runtime preloaded.  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_indexed_sparse_zha_amd", "csrc")
OUT = os.path.join(ROOT, "tree_indexed_sparse_zha_amd", "_build", "san")
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs ROCm's hipcc")
def test_abi_checks_are_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libzha.so")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-x", "hip", os.path.join(CSRC, "zha_api.cpp"),
           os.path.join(ROOT, "tests", "native", "launch_stubs.cpp"),
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stderr[-4000:]}"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=97",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98",
        "ZHA_LIB_PATH": lib,
        "PYTHONPATH": ROOT,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
    shutil.rmtree(OUT, ignore_errors=True)
