"""The allocation-free linear (convrot_w8a8_linear_noalloc) against the
linear with a caller workspace (convrot_w8a8_linear), through the C ABI:
bit for bit the same output on two calls in a row, the second with a
smaller input (the scratch area keeps the first call's contents), and the
oracle's bar on sampled outputs.  Run last: it leaves the scratch area in
use by nothing."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_rel_l2, bf16_from_dev, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(lib, M, K, N, seed):
    import torch
    say(f"noalloc linear M={M} K={K} N={N}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=seed)
    w = wl.make_weight(N, K, seed=seed)
    wq, ws = lib.quantize_weight(to_dev(w))
    xd = bf16_to_dev(x)
    y_ref = bf16_from_dev(lib.w8a8_linear(xd, wq, ws))
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = lib.convrot_w8a8_linear_noalloc(xd, M, K, wq, ws, N, 256, y)
    torch.cuda.synchronize()
    assert rc == 0, lib.convrot_status_string(rc)
    got = bf16_from_dev(y)
    assert np.array_equal(got, y_ref)
    # and the oracle's bar on sampled tokens x rows
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(M, min(M, 16), replace=False))
    rows = np.sort(rng.choice(N, min(N, 64), replace=False))
    xq_r, xs_r = oracle.rotate_quant(x[toks], 256)
    wq_r, ws_r = oracle.quantize_weight_i8(w[rows], 256)
    assert_rel_l2(got[np.ix_(toks, rows)], oracle.epilogue(oracle.gemm_i8(xq_r, wq_r), xs_r, ws_r))


def test_noalloc_matches_workspace_linear_twice(lib):
    _case(lib, 512, 4096, 4096, seed=11)   # first call: 2 MB of codes in the scratch area
    _case(lib, 37, 1024, 300, seed=12)     # second, smaller: the first call's bytes are still there


def test_noalloc_rejects_inputs_past_the_scratch_area(lib):
    import torch
    K = 4096
    M = lib.NOALLOC_SCRATCH_BYTES // K          # codes alone fill the area; the scales do not fit
    assert lib.convrot_workspace_size(M, K) > lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((64, K), dtype=torch.int8, device="cuda")
    ws = torch.zeros((64,), dtype=torch.float32, device="cuda")
    y = torch.full((M, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    rc = lib.convrot_w8a8_linear_noalloc(x, M, K, wq, ws, 64, 256, y)
    torch.cuda.synchronize()
    assert rc == 9                                # CONVROT_ERR_SCRATCH, nothing enqueued
    assert bool((y == 3.0).all())
