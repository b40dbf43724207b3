"""The Python binding refuses mismatched tensors before anything reaches the
library (no GPU needed: the tensors here are on the CPU, and a call whose
arguments all match fails only at the final device check, which proves every
shape, dtype and size check ran first)."""
import os

import pytest
import torch

import w8a8_quantized_linear_amd as cr


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(cr.library_path()):
        pytest.skip("libconvrot.so not built (run __graft_entry__.build())")
    cr.load()


M, K, N = 8, 512, 64


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i8(*shape):
    return torch.zeros(shape, dtype=torch.int8)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


ON_GPU = "must be on the GPU"


def test_w8a8_linear_checks():
    raises(ON_GPU, cr.w8a8_linear, bf(M, K), i8(N, K), f32(N))                 # all good: only the device fails
    raises("wq has shape", cr.w8a8_linear, bf(M, K), i8(N, K + 16), f32(N))    # K mismatch
    raises("wq has dtype", cr.w8a8_linear, bf(M, K), u8(N, K), f32(N))         # uint8 passed as int8 weights
    raises("wq has shape", cr.w8a8_linear, bf(M, K), u8(N, K // 2), f32(N))    # an int4 weight
    raises("scale has shape", cr.w8a8_linear, bf(M, K), i8(N, K), f32(N - 1))
    raises("scale has dtype", cr.w8a8_linear, bf(M, K), i8(N, K), torch.zeros(N, dtype=torch.float64))
    raises("out has shape", cr.w8a8_linear, bf(M, K), i8(N, K), f32(N), out=bf(M, N + 1))
    raises("out has dtype", cr.w8a8_linear, bf(M, K), i8(N, K), f32(N), out=f32(M, N))
    raises("workspace of", cr.w8a8_linear, bf(M, K), i8(N, K), f32(N), ws=u8(100))
    raises("1-D uint8", cr.w8a8_linear, bf(M, K), i8(N, K), f32(N), ws=f32(10000))
    raises("x must be 2-D", cr.w8a8_linear, bf(M * K), i8(N, K), f32(N))
    with pytest.raises(TypeError, match="bfloat16"):
        cr.w8a8_linear(f32(M, K), i8(N, K), f32(N))


def test_w4a8_linear_checks():
    raises(ON_GPU, cr.w4a8_linear, bf(M, K), u8(N, K // 2), f32(N))
    raises("wq4 has shape", cr.w4a8_linear, bf(M, K), u8(N, K), f32(N))
    raises("wq4 has dtype", cr.w4a8_linear, bf(M, K), i8(N, K // 2), f32(N))


def test_gemm_checks():
    raises(ON_GPU, cr.gemm_i8, i8(M, K), f32(M), i8(N, K), f32(N))
    raises("x_scale has shape", cr.gemm_i8, i8(M, K), f32(M + 1), i8(N, K), f32(N))
    raises("xq has dtype", cr.gemm_i8, u8(M, K), f32(M), i8(N, K), f32(N))
    raises("wq has shape", cr.gemm_i8, i8(M, K), f32(M), u8(N, K), f32(N), wbits=4)
    raises("wq has shape", cr.gemm_i8, i8(M, K), None, i8(N, K - 16), None, want_y=False)
    raises(ON_GPU, cr.gemm_i8, i8(M, K), None, i8(N, K), None, want_y=False)
    raises(ON_GPU, cr.gemm_bf16, bf(M, K), bf(N, K))
    raises("w has shape", cr.gemm_bf16, bf(M, K), bf(N, K + 16))
    raises("out has shape", cr.gemm_bf16, bf(M, K), bf(N, K), out=bf(N, M))


def test_multi_checks():
    good = [(i8(N, K), f32(N)), (i8(2 * N, K), f32(2 * N))]
    raises(ON_GPU, cr.linear_multi, bf(M, K), good)
    raises("weights\\[1\\] has shape", cr.linear_multi, bf(M, K), [good[0], (i8(N, K + 16), f32(N))])
    raises("weights\\[0\\] scale has shape", cr.linear_multi, bf(M, K), [(i8(N, K), f32(2 * N))])
    raises("outs\\[1\\] has shape", cr.linear_multi, bf(M, K), good, outs=[bf(M, N), bf(M, N)])
    raises("1..8 weights", cr.linear_multi, bf(M, K), good * 5)
    raises(ON_GPU, cr.gemm_i8_multi, i8(M, K), f32(M), good)
    raises("x_scale has shape", cr.gemm_i8_multi, i8(M, K), f32(1), good)


def test_norm_rotate_dequant_checks():
    raises(ON_GPU, cr.rotate_quant, bf(M, K))
    raises("x must be 2-D", cr.rotate_quant, bf(M, K, 1))
    raises(ON_GPU, cr.rmsnorm_rotate_quant, bf(M, K), f32(K))
    raises("norm_w has shape", cr.rmsnorm_rotate_quant, bf(M, K), f32(K - 1))
    raises("norm_w has dtype", cr.rmsnorm_rotate_quant, bf(M, K), bf(K))
    raises(ON_GPU, cr.dequantize_weight, i8(N, K), f32(N), K)
    raises("wq has shape", cr.dequantize_weight, i8(N, K), f32(N), 2 * K)       # K given separately
    raises("wq has shape", cr.dequantize_weight, i8(N, K), f32(N), K, wbits=4)
    raises(ON_GPU, cr.dequant_linear, bf(M, K), i8(N, K), f32(N))
    raises("out has shape", cr.dequant_linear, bf(M, K), i8(N, K), f32(N), out=bf(M, 1))
    raises(ON_GPU, cr.quantize_weight, f32(N, K))
    raises("even K", cr.quantize_weight, f32(N, K + 1), bits=4)


def test_raw_mirrors_check_buffer_sizes():
    """The C-named mirrors take explicit sizes; a buffer smaller than the
    bytes the call would touch is refused before the call."""
    ws = cr.convrot_workspace_size(M, K)
    raises("x holds", cr.convrot_w8a8_linear, bf(M, K - 16), M, K, i8(N, K), f32(N), N, 256, bf(M, N), u8(ws), ws)
    raises("y holds", cr.convrot_w8a8_linear, bf(M, K), M, K, i8(N, K), f32(N), N, 256, bf(M, N - 1), u8(ws), ws)
    raises("workspace holds", cr.convrot_w8a8_linear, bf(M, K), M, K, i8(N, K), f32(N), N, 256, bf(M, N),
           u8(ws), ws + 1)
    raises("wq holds", cr.convrot_w4a8_linear, bf(M, K), M, K, u8(N, K // 2 - 1), f32(N), N, 256, bf(M, N),
           u8(ws), ws)
    raises("acc_out holds", cr.convrot_gemm_i8, i8(M, K), f32(M), i8(N, K), 8, f32(N), M, N, K, f32(M, N - 1), None)
    raises("xq holds", cr.convrot_rotate_quant, bf(M, K), M, K, 256, i8(M, K - 1), f32(M))
    raises("norm_w holds", cr.convrot_rmsnorm_rotate_quant, bf(M, K), f32(K - 1), 1e-6, M, K, 256, i8(M, K), f32(M))
    raises("w_out holds", cr.convrot_dequantize_weight, i8(N, K), 8, f32(N), N, K, 256, bf(N, K - 1))
    raises("y holds", cr.convrot_gemm_i8_multi, i8(M, K), f32(M), 8, M, K, [(i8(N, K), f32(N), N, None, bf(1))])
    raises(ON_GPU, cr.convrot_w8a8_linear, bf(M, K), M, K, i8(N, K), f32(N), N, 256, bf(M, N), u8(ws), ws)
