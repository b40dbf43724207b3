"""Degenerate inputs through the C ABI on the GPU: empty batches (M = 0 and
N = 0 where allowed) for every entry point, and all-zero rows end to end."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_from_dev, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_empty_batches_are_no_ops(lib):
    import torch
    say("empty batches through every entry point")
    dev = "cuda"
    K, N = 512, 64
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    xq0 = torch.empty((0, K), dtype=torch.int8, device=dev)
    xs0 = torch.empty((0,), dtype=torch.float32, device=dev)
    w = torch.from_numpy(wl.make_weight(N, K, seed=1)).to(dev)
    wq, ws = lib.quantize_weight(w)
    y0 = torch.empty((0, N), dtype=torch.bfloat16, device=dev)
    nw = torch.zeros(K, dtype=torch.float32, device=dev)
    wsp = lib.workspace(1, K)
    assert lib.convrot_rotate_quant(x0, 0, K, 256, xq0, xs0) == 0
    assert lib.convrot_rmsnorm_rotate_quant(x0, nw, 1e-6, 0, K, 256, xq0, xs0) == 0
    assert lib.convrot_w8a8_linear(x0, 0, K, wq, ws, N, 256, y0, wsp, wsp.numel()) == 0
    assert lib.convrot_gemm_i8(xq0, xs0, wq, 8, ws, 0, N, K, None, y0) == 0
    assert lib.convrot_gemm_i8_multi(xq0, xs0, 8, 0, K, [(wq, ws, N, None, y0)]) == 0
    assert lib.convrot_linear_multi(x0, 0, K, 256, 8, [(wq, ws, N, None, y0)], wsp, wsp.numel()) == 0
    assert lib.convrot_gemm_bf16(x0, torch.zeros((N, K), dtype=torch.bfloat16, device=dev), 0, N, K, y0) == 0
    assert lib.convrot_dequant_linear(x0, 0, K, wq, 8, ws, N, 256, y0, wsp, wsp.numel()) == 0
    w_empty = torch.empty((0, K), dtype=torch.float32, device=dev)
    assert lib.convrot_quantize_weight(w_empty, 0, 0, K, 256, 8, torch.empty((0, K), dtype=torch.int8, device=dev),
                                       torch.empty((0,), dtype=torch.float32, device=dev)) == 0
    assert lib.convrot_dequantize_weight(torch.empty((0, K), dtype=torch.int8, device=dev), 8, xs0, 0, K, 256,
                                         torch.empty((0, K), dtype=torch.bfloat16, device=dev)) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("K,g", [(4096, 256), (1152, 16), (512, 1)])
def test_zero_rows_end_to_end(lib, K, g):
    """All-zero tokens quantize to scale 0 and codes 0 and give exactly zero
    outputs, while their neighbours are untouched (each token is independent)."""
    import torch
    say(f"zero rows end to end K={K} group={g}")
    M, N = 40, 96
    x = wl.make_activations(M, K, max(1, K // 100), seed=K)
    x[[0, 17, M - 1]] = 0
    w = wl.make_weight(N, K, seed=K)
    wq, ws = lib.quantize_weight(torch.from_numpy(w).cuda(), group=g)
    y = bf16_from_dev(lib.w8a8_linear(bf16_to_dev(x), wq, ws, group=g))
    assert np.all(y[[0, 17, M - 1]] == 0)
    wq_ref, ws_ref = oracle.quantize_weight_i8(w, g)
    y_ref = oracle.w8a8_linear(x, wq_ref, ws_ref, g)
    keep = np.setdiff1d(np.arange(M), [0, 17, M - 1])
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(f(y[keep]) - f(y_ref[keep])) / np.linalg.norm(f(y_ref[keep]))
    assert rel <= 1e-3
