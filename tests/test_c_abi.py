"""The C ABI from plain C: tests/c/abi_host_check.c is compiled with the host C compiler
against include/tp_linear.h, linked with the built libtp_linear.so, and run.  It makes only
calls that need no GPU (shape queries, argument validation, the loader's error path)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "tensor_sharded_linear_amd")
ROCM_INCLUDE = "/opt/rocm/include"


def test_plain_c_program_uses_the_abi(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("no host C compiler or ROCm headers")
    assert os.path.exists(os.path.join(LIB_DIR, "libtp_linear.so")), "build the library first"
    exe = str(tmp_path / "abi_host_check")
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-L", LIB_DIR, "-ltp_linear",
                    "-Wl,-rpath," + LIB_DIR, "-o", exe], check=True, capture_output=True, text=True, timeout=120)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host check: 16 checks ok" in r.stdout, r.stdout
