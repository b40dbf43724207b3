"""Group-256 rotate-quantize over every row length the fast kernel takes
(K = 256 * G for G = 1..64, with the unused group slots of a wave masked),
plain and with the fused RMSNorm, on both sides of the few-tokens split."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_codes_close, assert_scales_close, bf16_from_dev, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

# Row lengths of common hidden and MLP widths that are multiples of 256 but
# not of 1024 (2560, 3584, 5120, 9728, 13824), the edges of every
# waves-per-token band (4, 5, 16, 17, 32, 33, 48, 49, 64 groups), and both
# token counts (below 4096 a token is split over twice the waves).
KS = [256, 512, 1280, 2560, 3584, 4096, 4352, 5120, 8192, 8448, 9728, 12288, 12544, 13824, 16384]


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("M", [37, 4099])
def test_rotate_quant_g256_all_widths(lib, M, K):
    if M * K > 4099 * 8192:
        M = 700                       # keep the oracle's dense product to seconds
    say(f"rotate_quant g256 M={M} K={K}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M + 3 * K)
    xq, xs = lib.rotate_quant(bf16_to_dev(x))
    xq_ref, xs_ref = oracle.rotate_quant(x, 256)
    assert_scales_close(xs.cpu().numpy(), xs_ref)
    assert_codes_close(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("K", [256, 1280, 2560, 5120, 9728, 13824])
@pytest.mark.parametrize("M", [21, 4100])
def test_rmsnorm_rotate_quant_all_widths(lib, M, K):
    if M * K > 4100 * 5120:
        M = 600
    say(f"rmsnorm_rotate_quant g256 M={M} K={K}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M + 5 * K)
    w = wl.make_norm_weight(K, max(1, K // 100), seed=K)
    xq, xs, y = lib.rmsnorm_rotate_quant(bf16_to_dev(x), to_dev(w), want_y=True)
    xq_ref, xs_ref, y_ref = oracle.rmsnorm_rotate_quant(x, w)
    assert np.array_equal(bf16_from_dev(y), y_ref)
    assert_scales_close(xs.cpu().numpy(), xs_ref)
    assert_codes_close(xq.cpu().numpy(), xq_ref)


def test_masked_slots_write_nothing(lib):
    """K = 2560 fills 10 of a wave's 12 group slots: the codes buffer past
    each row's end (the next row) must hold exactly that row's codes, and a
    guard region after the last row stays untouched."""
    import torch
    M, K = 9, 2560
    say("rotate_quant g256 masked slots")
    x = wl.make_activations(M, K, 25, seed=8)
    xq = torch.full((M * K + 4096,), 0x5a, dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    assert lib.convrot_rotate_quant(bf16_to_dev(x), M, K, 256, xq[:M * K], xs) == 0
    torch.cuda.synchronize()
    h = xq.cpu().numpy()
    xq_ref, _ = oracle.rotate_quant(x, 256)
    assert_codes_close(h[:M * K].reshape(M, K), xq_ref)
    assert np.all(h[M * K:] == 0x5a)
