"""Build libconvrot.so (HIP, gfx950) in-tree with hipcc.

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into one shared library next to this file.  Usage:
    python -m w8a8_quantized_linear_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libconvrot.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    _check_defined(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def _check_defined(lib: str) -> None:
    """Fail the build if the library leaves any of its own symbols undefined
    (for instance a kernel's host-side stub that the compiler did not emit):
    such a library would only fail later, when it is loaded."""
    nm = shutil.which("nm")
    if nm is None:
        return
    r = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [line.split()[-1] for line in r.stdout.splitlines() if "convrot" in line]
    if missing:
        os.remove(lib)
        raise RuntimeError("link left library symbols undefined:\n  " + "\n  ".join(missing))


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
