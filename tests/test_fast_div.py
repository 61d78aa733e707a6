"""The invariant-divisor division the fused RoPE kernel uses to find a row's
token (FastDiv in csrc/fnorm_device.hpp), checked on the host against plain
integer division: tests/c_abi/fast_div_check.cpp includes the kernels' own
header, so the code checked is the code the kernels compile (CPU only)."""
import os
import shutil
import subprocess

import pytest

from transformer_row_normalization_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fast_div_matches_integer_division(tmp_path):
    hipcc = shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "fast_div_check"
    subprocess.run([hipcc, "-O2", "-std=c++17", f"--offload-arch={_build.ARCH}",
                    "-Wno-unused-command-line-argument",
                    os.path.join(ROOT, "tests", "c_abi", "fast_div_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
