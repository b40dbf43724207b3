"""GPU parity of the small-group fast path (group 16, the ConvRot vision
group size for widths 1152 and 4304, and group 1) against the oracle."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import (assert_codes_close, assert_codes_off_ties, assert_rel_l2, assert_scales_close,
                               bf16_from_dev, bf16_to_dev, exact_quotients, say, to_dev)
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

# K values cover every rows-per-wave choice (1, 2 and 4 rows of a wave) and
# 1..8 chunks per lane, plus the generic kernel just past the fast path.
SHAPES = [(1, 16), (7, 48), (33, 1152), (9, 4304), (64, 4096), (5, 8192), (3, 8208), (100, 528), (257, 2048),
          (3, 1040), (20, 3072), (4096, 1152)]


@pytest.mark.parametrize("g", [16, 1])
@pytest.mark.parametrize("M,K", SHAPES)
def test_small_group_rotate_quant(lib, g, M, K):
    say(f"rotate_quant small group={g} M={M} K={K}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M + K + g)
    xq, xs = lib.rotate_quant(bf16_to_dev(x), group=g)
    xq_ref, xs_ref = oracle.rotate_quant(x, g)
    assert_scales_close(xs.cpu().numpy(), xs_ref)
    assert_codes_close(xq.cpu().numpy(), xq_ref)
    if g == 1 and M * K <= 1 << 20:
        # no rotation: the inputs are exact, so a code can differ only where
        # the fp32 quotient rounds across a boundary n + 1/2
        q_exact = exact_quotients(wl.bf16_bits_to_float(x), xs_ref, 1)
        assert_codes_off_ties(xq.cpu().numpy(), xq_ref, q_exact)


@pytest.mark.parametrize("g", [16, 1])
def test_small_group_special_rows(lib, g):
    """Zero rows, exact half-integer quotients (ties away from zero), tiny and
    huge rows, one-hot rows."""
    say(f"rotate_quant small group={g} special rows")
    K = 1152
    x = np.zeros((8, K), dtype=np.float32)
    x[1, 3] = 1.0
    x[2, :16] = [127.0, 0.5, -0.5, 1.5, -2.5] + [0.0] * 11 if g == 1 else 0.0
    x[3] = 1e-33
    x[4, ::9] = 2.0 ** 100
    x[5] = np.linspace(-3, 3, K)
    x[6, 100:116] = 0.75
    x[7] = wl.bf16_bits_to_float(wl.make_activations(1, K, 11, seed=3))[0]
    if g == 16:
        # a group whose transform is (127, 0.5, -0.5, 0, ...) * 4: ties at +-0.5
        import scipy.linalg
        v = np.zeros(16)
        v[0], v[1], v[2] = 127.0, 0.5, -0.5
        x[2, :16] = v @ (scipy.linalg.hadamard(16) / 4.0)
    xb = wl.float_to_bf16_bits(x)
    xq, xs = lib.rotate_quant(bf16_to_dev(xb), group=g)
    xq, xs = xq.cpu().numpy(), xs.cpu().numpy()
    xq_ref, xs_ref = oracle.rotate_quant(xb, g)
    assert np.all(xq[0] == 0) and xs[0] == 0
    assert np.array_equal(xq[2, :16], xq_ref[2, :16])
    assert xq[2, 1] == 1 and xq[2, 2] == -1
    normal = xs_ref >= np.float32(2.0 ** -126)
    assert_scales_close(xs[normal], xs_ref[normal])
    # constructed rows (every sum exact in fp32) and the rest: the oracle's
    # codes except at rounding boundaries of the exact quotient
    q_exact = exact_quotients(wl.bf16_bits_to_float(xb), xs_ref, g)
    assert_codes_off_ties(xq[normal], xq_ref[normal], q_exact[normal])


@pytest.mark.parametrize("name,K,N", [("qkv", 1152, 3456), ("proj", 1152, 1152), ("fc1", 1152, 4304),
                                      ("fc2", 4304, 1152)])
def test_vision_linears_sampled(lib, name, K, N):
    """The vision block's linears with group 16 at M=4096 patches: sampled
    outputs against the oracle's full path."""
    import torch
    M = 4096
    say(f"vision {name} M={M} K={K} N={N} group 16")
    x = wl.make_activations(M, K, K // 100, seed=K + N)
    w = wl.make_weight(N, K, seed=N)
    wq, ws = lib.quantize_weight(torch.from_numpy(w).cuda(), group=16)
    y = bf16_from_dev(lib.w8a8_linear(bf16_to_dev(x), wq, ws, group=16))
    rng = np.random.default_rng(K + N)
    toks = np.sort(rng.choice(M, 12, replace=False))
    rows = np.sort(rng.choice(N, 96, replace=False))
    xq_ref, xs_ref = oracle.rotate_quant(x[toks], 16)
    wq_ref, ws_ref = oracle.quantize_weight_i8(w[rows], 16)
    y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref, wq_ref), xs_ref, ws_ref)
    assert_rel_l2(y[np.ix_(toks, rows)], y_ref)


def test_vision_w4a8_linear_sampled(lib):
    """Packed int4 weights with group 16 at the vision MLP shape (K = 1152,
    not a multiple of 256, so the GEMM takes its range-checked path)."""
    import torch
    M, K, N = 1024, 1152, 4304
    say(f"vision W4A8 M={M} K={K} N={N} group 16")
    x = wl.make_activations(M, K, K // 100, seed=77)
    w = wl.make_weight(N, K, seed=78)
    wq4, ws = lib.quantize_weight(torch.from_numpy(w).cuda(), group=16, bits=4)
    y = bf16_from_dev(lib.w4a8_linear(bf16_to_dev(x), wq4, ws, group=16))
    rng = np.random.default_rng(79)
    toks = np.sort(rng.choice(M, 12, replace=False))
    rows = np.sort(rng.choice(N, 96, replace=False))
    packed_ref, ws_ref, _ = oracle.quantize_weight_i4(w[rows], 16)
    y_ref = oracle.w4a8_linear(x[toks], packed_ref, ws_ref, 16)
    assert_rel_l2(y[np.ix_(toks, rows)], y_ref)
