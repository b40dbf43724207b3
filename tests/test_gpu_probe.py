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
    import torch  # noqa: F401  (torch's HIP runtime must be the process's: see the binding's load())
    lib = ctypes.CDLL(LIB)
    for fn in (lib.mfma_rate_launch, lib.mfma_rate_launch_bf16):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    return lib


def test_probe_exports_launcher_and_rejects_bad_arguments():
    lib = _lib()
    assert lib.mfma_rate_launch(0, 1, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, -1, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, 1 << 20, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch(2, 1, None, None) == 1
    assert lib.mfma_rate_launch_bf16(0, 1, ctypes.c_void_p(0x1000), None) == 1
    assert lib.mfma_rate_launch_bf16(2, 1, None, None) == 1


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


@pytest.mark.gpu
def test_probe_bf16_loop_accumulates():
    """The bf16 loop's sums (fp32 accumulation of bf16 products in [1, 4))
    are finite, positive and grow with the iterations (the accumulation
    order inside an MFMA is the hardware's, so the doubling is checked to
    fp32 rounding, not exactly)."""
    import torch
    lib = _lib()
    blocks = 8
    out = torch.zeros((blocks * 256,), dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sums = []
    for iters in (1, 2):
        print(f"mfma probe bf16: {blocks} workgroups, {iters} iterations", flush=True)
        assert lib.mfma_rate_launch_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), stream) == 0
        torch.cuda.synchronize()
        sums.append(out.view(torch.float32).double().clone())
    assert torch.isfinite(sums[1]).all() and (sums[0] > 0).all()
    assert torch.allclose(sums[1], 2 * sums[0], rtol=1e-5)


STREAM = os.path.join(HERE, "gpu_probe", "libstream_rq.so")


def _stream():
    if not os.path.exists(STREAM):
        pytest.skip("tests/gpu_probe/libstream_rq.so not built (run __graft_entry__.build())")
    import torch  # noqa: F401  (as in _lib)
    fn = ctypes.CDLL(STREAM).stream_rq_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def test_stream_probe_rejects_bad_arguments():
    fn = _stream()
    p = ctypes.c_void_p(0x1000)
    assert fn(None, p, p, 4, 256, 0, 8, None) == 1
    assert fn(p, p, p, 0, 256, 0, 8, None) == 1
    assert fn(p, p, p, 4, 250, 0, 8, None) == 1      # K not a multiple of 16
    assert fn(p, p, p, 4, 256, 2, 8, None) == 1      # no such mode
    assert fn(p, p, p, 4, 256, 1, 0, None) == 1      # empty grid
    assert fn(ctypes.c_void_p(0x1008), p, p, 4, 256, 0, 8, None) == 1  # misaligned


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1])
def test_stream_probe_moves_every_byte(mode):
    """Both launch shapes write the high byte of every bf16 word and one word
    per row: the probe really reads all of its input."""
    import torch
    fn = _stream()
    M, K = 37, 4096 + 256
    x = torch.randint(-32768, 32768, (M, K), dtype=torch.int32, device="cuda").to(torch.int16)
    q = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    v = torch.zeros((M,), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert fn(x.data_ptr(), q.data_ptr(), v.data_ptr(), M, K, mode, 5, stream) == 0
    torch.cuda.synchronize()
    expect = ((x.to(torch.int32) >> 8) & 0xff).to(torch.uint8)
    assert torch.equal(q, expect)
    assert torch.equal(v, torch.ones_like(v))
