"""The library's host code (pool metadata, argument checks, batch and split
planning, shared-prefix grouping) and the CPU oracle, built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only; the
device launchers are stubs that abort if reached) and run over seeded random
operation sequences with the two pools' states compared after every
operation (tests/c/sanitize_host.cpp).  CPU only."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_gqa_layer_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not gcc or not gxx or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc/g++ or the ROCm headers are missing")
    obj = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "sanitize_host")
    subprocess.check_call([gcc, *SAN, "-std=c11", "-c",
                           os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-o", obj])
    subprocess.check_call([gxx, *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                           "-I", CSRC, os.path.join(ROOT, "tests", "c", "sanitize_host.cpp"),
                           os.path.join(CSRC, "pool_meta.cpp"), os.path.join(CSRC, "api.cpp"),
                           obj, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                           "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe, "40"], env=env, capture_output=True, text=True, timeout=900)
    assert p.returncode == 0, (p.stdout + p.stderr)[-4000:]
    assert "no mismatch" in p.stdout
