"""Build the measurement helpers under tests/gpu_probe/ (gfx950, hipcc) next
to their sources.  They are not part of the library: bench.py's
--profile mfma_rate and its mfma_loop context line load them."""
import os
import subprocess

from w8a8_quantized_linear_amd import build as lib_build

HERE = os.path.dirname(os.path.abspath(__file__))
MFMA_RATE = os.path.join(HERE, "libmfma_rate.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "mfma_rate.hip")
    tmp = MFMA_RATE + ".tmp%d" % os.getpid()
    cmd = [lib_build.HIPCC, *lib_build.COMMON, "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, MFMA_RATE)
    if verbose:
        print(f"built {MFMA_RATE}")
    return MFMA_RATE
