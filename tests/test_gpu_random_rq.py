"""Rotate-quantize on irregular shapes (fixed list): group 256 (the fast path
at every waves-per-token band), group 16 and group 1 (the small-group
kernel), plain and with the fused RMSNorm; codes and scales on sampled
tokens against the oracle, and guard words around the code and scale
buffers untouched."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_codes_close, assert_scales_close, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

# (M, K, group, fused norm)
SHAPES = [
    (1, 256, 256, False), (3001, 2560, 256, False), (4095, 4352, 256, False), (4097, 4096, 256, False),
    (777, 12544, 256, False), (12, 16384, 256, False), (2049, 1152, 16, False), (333, 4304, 16, False),
    (5000, 8192, 16, False), (4099, 512, 1, False), (17, 8000, 1, False), (999, 3328, 256, True),
    (4100, 6400, 256, True), (5, 16384, 256, True), (4103, 3328, 256, True),
]
GUARD = 256


@pytest.mark.parametrize("M,K,g,fused", SHAPES)
def test_rotate_quant_irregular(lib, M, K, g, fused):
    import torch
    say(f"{'rmsnorm_' if fused else ''}rotate_quant irregular M={M} K={K} group={g}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M + K + g)
    qbuf = torch.full((GUARD + M * K + GUARD,), 0x5a, dtype=torch.int8, device="cuda")
    sbuf = torch.full((GUARD + M + GUARD,), -7.0, dtype=torch.float32, device="cuda")
    xq, xs = qbuf[GUARD:GUARD + M * K], sbuf[GUARD:GUARD + M]
    if fused:
        w = wl.make_norm_weight(K, max(1, K // 100), seed=K)
        rc = lib.convrot_rmsnorm_rotate_quant(bf16_to_dev(x), to_dev(w), 1e-6, M, K, g, xq, xs, None)
    else:
        rc = lib.convrot_rotate_quant(bf16_to_dev(x), M, K, g, xq, xs)
    torch.cuda.synchronize()
    assert rc == 0
    qh, sh = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(qh[:GUARD] == 0x5a) and np.all(qh[GUARD + M * K:] == 0x5a)
    assert np.all(sh[:GUARD] == -7.0) and np.all(sh[GUARD + M:] == -7.0)
    rng = np.random.default_rng(M + K)
    toks = np.unique(np.concatenate([rng.choice(M, min(M, 48), replace=False), [0, M - 1]]))
    if fused:
        q_ref, s_ref, _ = oracle.rmsnorm_rotate_quant(x[toks], w, eps=1e-6, group=g)
    else:
        q_ref, s_ref = oracle.rotate_quant(x[toks], g)
    assert_scales_close(sh[GUARD:GUARD + M][toks], s_ref)
    assert_codes_close(qh[GUARD:GUARD + M * K].reshape(M, K)[toks], q_ref)
