"""The boundary is a plain C ABI: a C program built with gcc against
include/pkv.h and the library runs the pool's known answers (no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "paged_kv_gqa_layer_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_against_the_header(tmp_path):
    exe = tmp_path / "abi_host"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", LIBDIR, "-lpkv",
                    "-Wl,-rpath," + LIBDIR, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
