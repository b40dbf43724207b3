"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two programs, each built in a temporary directory with the sanitizers on and
run with leak detection:
- the CPU oracle (gcc) driven by tests/host/oracle_sanitize.c over every
  exported function, its edge cases and rejected arguments;
- the library's host side (hipcc, sanitizers on the host pass only; the
  device code is built as usual and never runs here) driven by
  tests/host/abi_from_c.c, which goes through every argument check of the
  C ABI without a GPU.
Any sanitizer report makes the program exit non-zero (no recovery).
"""
import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess

import pytest

from w8a8_quantized_linear_amd import build as lib_build

ROOT = pathlib.Path(__file__).resolve().parent.parent
HOST = ROOT / "tests" / "host"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = pathlib.Path(ROCM) / "llvm" / "bin"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, expect):
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=SAN_ENV)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert expect in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           *SAN, str(ROOT / "oracle" / "convrot_oracle.c"), str(HOST / "oracle_sanitize.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    _run(exe, "oracle sanitizer checks passed")


@pytest.mark.skipif(not (pathlib.Path(lib_build.HIPCC).exists() and (CLANG / "clang++").exists()),
                    reason="hipcc / ROCm clang not available")
def test_library_host_validation_under_asan_ubsan(tmp_path):
    # Sanitizers on the host pass only: each -fsanitize option goes through
    # -Xarch_host, so the device code is compiled exactly as in the library.
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]

    def compile_one(src):
        obj = tmp_path / (pathlib.Path(src).name + ".o")
        cmd = [lib_build.HIPCC, *lib_build.COMMON, "-g", *host_san, "-c", src, "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return str(obj)

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, lib_build.sources()))
    drv = tmp_path / "abi_from_c.o"
    subprocess.run([str(CLANG / "clang"), "-std=c11", "-g", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", str(ROOT / "include"), "-I", f"{ROCM}/include", "-c", str(HOST / "abi_from_c.c"),
                    "-o", str(drv)], check=True, capture_output=True, text=True)
    exe = tmp_path / "abi_sanitize"
    subprocess.run([str(CLANG / "clang++"), *SAN, str(drv), *objs, f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)], check=True, capture_output=True, text=True)
    _run(exe, "C ABI checks passed")
