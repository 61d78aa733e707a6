"""The library's host code under AddressSanitizer and UBSan (CPU only).

fnorm_api.hip (argument validation, overlap checks, kernel tables, the
candidate cache, error text) is rebuilt with the sanitizers on its host
code only (-Xarch_host), linked with the kernel objects of the normal
build, and driven by tests/c_abi/host_paths.c through every path that
needs no GPU.  Any sanitizer report, leak or wrong status fails the test.
"""
import os
import shutil
import subprocess

import pytest

import transformer_row_normalization_amd as trn
from transformer_row_normalization_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
KERNEL_OBJECTS = [s.replace(".hip", ".o") for s in _build.SOURCES if s != "fnorm_api.hip"]


def test_host_paths_under_asan_and_ubsan(tmp_path):
    objdir = os.path.join(os.path.dirname(trn.LIB_PATH), "_build")
    objs = [os.path.join(objdir, o) for o in KERNEL_OBJECTS]
    if shutil.which("hipcc") is None or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang not available")
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, f"kernel objects missing (run the build first): {missing}"
    api = tmp_path / "api_san.o"
    drv = tmp_path / "host_paths.o"
    exe = tmp_path / "host_paths"
    subprocess.run([shutil.which("hipcc"), "-O1", "-g", f"--offload-arch={_build.ARCH}",
                    "-std=c++17", "-fPIC", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Wno-unused-command-line-argument", f"-I{_build.INCLUDE}",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(_build.CSRC, "fnorm_api.hip"), "-o", str(api)],
                   check=True, capture_output=True)
    subprocess.run([CLANG, "-std=c11", "-g", "-Wall", "-Wextra", "-Werror",
                    "-fsanitize=address,undefined", f"-I{_build.INCLUDE}", "-c",
                    os.path.join(ROOT, "tests", "c_abi", "host_paths.c"), "-o", str(drv)],
                   check=True, capture_output=True)
    rocm_lib = "/opt/rocm/lib"
    subprocess.run([CLANG + "++", "-fsanitize=address,undefined", "-o", str(exe), str(drv),
                    str(api), *objs, f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert "host paths ok" in out.stdout
    assert "runtime error" not in out.stderr and "AddressSanitizer" not in out.stderr
