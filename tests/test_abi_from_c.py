"""The C header compiles as plain C11 and the library links and answers
from a C program (no GPU needed: only validation paths are exercised)."""
import os
import pathlib
import shutil
import subprocess

import pytest

import w8a8_quantized_linear_amd as cr

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = ROOT / "tests" / "host" / "abi_from_c.c"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def test_c_program_links_and_validates(tmp_path):
    lib = pathlib.Path(cr.library_path())
    if not lib.exists():
        pytest.skip("libconvrot.so not built")
    exe = tmp_path / "abi_from_c"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", str(ROOT / "include"), "-I", f"{ROCM}/include", str(SRC), "-o", str(exe),
           "-L", str(lib.parent), "-lconvrot", f"-Wl,-rpath,{lib.parent}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "C ABI checks passed" in res.stdout
