"""The C-ABI validation layer under AddressSanitizer and UndefinedBehaviorSanitizer.

mxq_api.hip is compiled with both sanitizers on its host code only (device code is never
instrumented), linked with the library's other objects and tests/sanitize/abi_checks.cpp,
a driver that takes every entry point through its argument checks (sizes and pitches up
to the int64 limits, NULL and misaligned pointers, unknown enums), the host-only FP8
scale and workspace functions and empty problems.  None of those calls reaches the GPU.
UndefinedBehaviorSanitizer runs without recovery, so a signed overflow in a size check
fails the test.  CPU only.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_microscaled_quantization_amd")
sys.path.insert(0, PKG)

import build  # noqa: E402

CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-2000:] + r.stderr[-4000:]
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_abi_validation_under_host_sanitizers(tmp_path):
    objdir = os.path.join(PKG, "_build")
    others = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in build.SOURCES if s != "mxq_api.hip"]
    if not all(os.path.exists(o) for o in others):
        build.build()
    api_obj = str(tmp_path / "mxq_api_san.o")
    flags = [f for f in build.FLAGS if f != "-shared"]
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([build.hipcc(), *flags, "-O1", "-g", *host_san, "-c", "-o", api_obj, os.path.join(build.CSRC, "mxq_api.hip")])
    drv_obj = str(tmp_path / "abi_checks.o")
    _run([CLANG, "-std=c++17", "-O1", "-g", *SAN, "-c", "-o", drv_obj,
          os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")])
    exe = str(tmp_path / "abi_checks")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    _run([CLANG, *SAN, "-o", exe, drv_obj, api_obj, *others, "-L" + rocm_lib, "-lamdhip64",
          "-Wl,-rpath," + rocm_lib])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in out and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
