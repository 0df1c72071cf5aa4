"""Host-side helpers of bench.py (no GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_digest_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* another\n   header */\nint f(int x) {   return x + 1; }\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_code_digest(a) == bench.kernel_code_digest(b)
    assert bench.kernel_code_digest(a, c) != bench.kernel_code_digest(c, a)
    assert bench.kernel_code_digest(a) != bench.kernel_code_digest(c)


def test_percentiles():
    p = bench.pct([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p["p50"] == 3.0 and p["p10"] < p["p50"] < p["p90"]


def test_more_than_one_gpu_is_refused_before_any_device_work():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                           env=dict(os.environ, **env), capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""
