"""bench.py's contract checks that need no GPU: more than one GPU is
refused with a message, and the source hash that guards the recorded HBM
traffic ignores comments but not code."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    msg = json.loads(out.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_code_hash_ignores_comments_only():
    code = "int f(int a) {\n    return a + 1;  // one more\n}\n"
    same = "/* header */\nint f(int a) {\n\n    return a + 1;\n}\n// end\n"
    other = "int f(int a) {\n    return a + 2;\n}\n"
    assert bench._code_only(code) == bench._code_only(same)
    assert bench._code_only(code) != bench._code_only(other)
    assert len(bench.kernel_source_hash()) == 16
