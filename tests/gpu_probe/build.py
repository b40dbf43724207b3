"""Build the measurement helpers under tests/gpu_probe/ (gfx950, hipcc) next
to their sources.  They are not part of the library: bench.py's
--profile mfma_rate, its mfma_loop context line and its same-bytes
streaming reference beside the rotate-quantize passes load them."""
import os
import subprocess

from w8a8_quantized_linear_amd import build as lib_build

HERE = os.path.dirname(os.path.abspath(__file__))
MFMA_RATE = os.path.join(HERE, "libmfma_rate.so")
STREAM_RQ = os.path.join(HERE, "libstream_rq.so")


def _build_one(src_name: str, lib: str, verbose: bool) -> str:
    src = os.path.join(HERE, src_name)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [lib_build.HIPCC, *lib_build.COMMON, "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False) -> str:
    _build_one("stream_rq.hip", STREAM_RQ, verbose)
    return _build_one("mfma_rate.hip", MFMA_RATE, verbose)
