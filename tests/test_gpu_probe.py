"""The bench's MFMA-rate helper (tests/gpu_probe/mfma_rate.hip): it builds,
exports its launcher, and really does its MFMAs (doubling the iterations
doubles every lane's sum; zero iterations give zeros)."""
import ctypes
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_probe", "libmfma_rate.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("tests/gpu_probe/libmfma_rate.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.mfma_rate_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_rate_launch.restype = ctypes.c_int
    return lib


def test_probe_exports_launcher_and_rejects_bad_arguments():
    lib = _lib()
    assert lib.mfma_rate_launch(0, 1, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, -1, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, 1 << 20, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, 1, None, None) == 1


@pytest.mark.gpu
def test_probe_work_scales_with_iterations():
    import torch
    lib = _lib()
    blocks = 8
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sums = []
    for iters in (0, 1, 2, 3):
        print(f"mfma probe: {blocks} workgroups, {iters} iterations", flush=True)
        assert lib.mfma_rate_launch(blocks, iters, ctypes.c_void_p(out.data_ptr()), stream) == 0
        torch.cuda.synchronize()
        sums.append(out.clone())
    assert torch.count_nonzero(sums[0]) == 0
    assert torch.count_nonzero(sums[1]) > 0
    assert torch.equal(sums[2], sums[1] * 2) and torch.equal(sums[3], sums[1] * 3)
