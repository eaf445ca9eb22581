"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI layer (csrc/capi.cpp, csrc/workspace.cpp) built with g++ and run
  against launcher stubs that write every byte of each region a kernel would
  be handed: a workspace carved past the caller's buffer, or an output sized
  wrong, is a heap overflow (tests/sanitize/capi_host_check.cpp).
* The fp64 oracle (oracle/dsa_oracle.c) built with gcc and run on edge cases of
  every function (tests/sanitize/oracle_check.c).

Any sanitizer report aborts the program (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_gemm_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def _build_and_run(compile_cmd, exe, expect):
    c = _run(compile_cmd)
    assert c.returncode == 0, c.stdout + c.stderr
    r = _run([exe], env=ENV, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert expect in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP runtime API headers")
def test_capi_host_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "capi_check")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "capi_host_check.cpp"),
           os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "workspace.cpp"), "-o", exe]
    _build_and_run(cmd, exe, "capi host check ok")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    cmd = ["gcc", "-std=c99", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
           os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-lm", "-o", exe]
    _build_and_run(cmd, exe, "oracle check ok")
