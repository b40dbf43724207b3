"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Both sides receive the same seeded inputs from
w8a8_quantized_linear_amd.workloads (or seeded random codes); no expected
value is ever derived from a GPU result.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import (assert_clip_choice, assert_codes_close, assert_codes_off_ties, assert_rel_l2,
                               assert_scales_close, bf16_from_dev, bf16_to_dev, exact_quotients, say, to_dev)
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ GEMM

GEMM_SHAPES = [
    (1, 1, 16), (16, 256, 512), (33, 70, 208), (128, 128, 128), (130, 257, 272),
    (300, 200, 1040), (512, 4096, 4096), (7, 1024, 12288),
    (300, 200, 1152), (77, 130, 384),     # K a multiple of 128 but not 256 (unchecked loads, odd step count)
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i8_bit_exact(lib, M, N, K):
    say(f"gemm_i8 W8 M={M} N={N} K={K}")
    rng = np.random.default_rng(1000 + M + N + K)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    xs = (rng.random(M) * 0.1 + 1e-3).astype(np.float32)
    ws = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    acc, y = lib.gemm_i8(to_dev(a), to_dev(xs), to_dev(b), to_dev(ws), wbits=8)
    acc_ref = oracle.gemm_i8(a, b)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert np.array_equal(bf16_from_dev(y), oracle.epilogue(acc_ref, xs, ws))


@pytest.mark.parametrize("wbits,M,N,K", [
    (8, 2048, 6144, 2048),   # 256x192, persistent
    (8, 8704, 4096, 2048),   # 256x192, about three tiles per workgroup
    (8, 2048, 4096, 768),    # 128x128
    (8, 2048, 4096, 640),    # 128x128, K an odd number of 128-steps
    (8, 2048, 4096, 2048),   # 256x128 with three stages, one tile per CU
    (8, 1990, 4090, 2064),   # the same, ragged M, N and K
    (8, 512, 4000, 1040),    # 64x128 with four stages, ragged N and K
    (8, 1000, 4000, 1040),   # 128x128 with four stages, ragged M, N and K
    (8, 2000, 12280, 2048),  # 256x192, ragged M and N (N not a multiple of 8)
    (8, 8700, 12288, 256),   # 256x256, ragged M
    (4, 2048, 12288, 2048),  # packed int4, 256x192
    (4, 4000, 12288, 256),   # packed int4, 256x256, ragged M
    (4, 1990, 4090, 2080),   # packed int4, 256x128 with three stages, ragged M, N and K
    (4, 1000, 4000, 1056),   # packed int4, 128x128 with four stages
    (4, 512, 4000, 1056),    # packed int4, 64x128 with four stages
])
def test_gemm_i8_large_sampled(lib, wbits, M, N, K):
    """Shapes whose tile plan uses the large tiles (persistent or not),
    including ragged edges; int32 accumulators bit-exact on sampled rows
    (all columns) against an int64 product, bf16 outputs bit-exact against
    the oracle's epilogue."""
    say(f"gemm_i8 W{wbits} large M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K + wbits)
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    xs = (rng.random(M) * 0.1 + 1e-3).astype(np.float32)
    ws = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    if wbits == 8:
        b = rng.integers(-127, 128, (N, K), dtype=np.int8)
        wdev = to_dev(b)
    else:
        packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        b = oracle.unpack_i4(packed)
        wdev = to_dev(packed)
    acc, y = lib.gemm_i8(to_dev(a), to_dev(xs), wdev, to_dev(ws), wbits=wbits)
    rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False), [0, 255, 256, M - 1]]))
    ref = a[rows].astype(np.int64) @ b.astype(np.int64).T
    got = acc[rows.tolist()].cpu().numpy()
    assert np.array_equal(got, ref)
    yref = oracle.epilogue(ref.astype(np.int32), xs[rows], ws)
    assert np.array_equal(bf16_from_dev(y[rows.tolist()]), yref)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 256, 512), (33, 70, 224), (130, 257, 4096), (64, 12288, 4096),
                                   (130, 257, 1152)])
def test_gemm_w4_bit_exact(lib, M, N, K):
    say(f"gemm_i8 W4 M={M} N={N} K={K}")
    rng = np.random.default_rng(2000 + M + N + K)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b4 = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)   # every nibble value, -8..7
    xs = (rng.random(M) * 0.1 + 1e-3).astype(np.float32)
    ws = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    acc, y = lib.gemm_i8(to_dev(a), to_dev(xs), to_dev(b4), to_dev(ws), wbits=4)
    acc_ref = oracle.gemm_i8(a, oracle.unpack_i4(b4))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert np.array_equal(bf16_from_dev(y), oracle.epilogue(acc_ref, xs, ws))


def test_gemm_extreme_accumulators(lib):
    say("gemm_i8 extremes K=32768")
    K = 32768
    a = np.full((3, K), 127, dtype=np.int8)
    a[1] = -128
    a[2, ::2] = -127
    b = np.full((2, K), -128, dtype=np.int8)
    b[1] = 127
    acc, _ = lib.gemm_i8(to_dev(a), None, to_dev(b), None, wbits=8, want_y=False)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i8(a, b))


# ------------------------------------------------------- rotate + quantize

RQ_CASES = [
    (16, 512, 256), (1, 256, 256), (7, 4352, 256), (512, 4096, 256), (64, 12288, 256), (3, 32768, 256),
    (64, 4096, 1), (64, 4096, 16), (64, 4096, 2), (64, 4096, 128), (40, 1152, 16), (9, 4304, 16),
]


@pytest.mark.parametrize("M,K,g", RQ_CASES)
def test_rotate_quant_parity(lib, M, K, g):
    say(f"rotate_quant M={M} K={K} group={g}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M * 7 + K + g)
    xq, xs = lib.rotate_quant(bf16_to_dev(x), group=g)
    xq_ref, xs_ref = oracle.rotate_quant(x, g)
    assert_scales_close(xs.cpu().numpy(), xs_ref)
    assert_codes_close(xq.cpu().numpy(), xq_ref)


def test_rotate_quant_special_rows(lib):
    say("rotate_quant special rows")
    K = 1024
    x = np.zeros((6, K), dtype=np.float32)
    x[1, 37] = 1.0                      # one-hot: all codes +-127
    x[2, 256:512] = 0.75                # constant group: a single 127
    x[3] = 1e-30                        # tiny (bf16 keeps it normal)
    x[4, ::3] = -3.0
    x[5] = np.linspace(-100, 100, K)
    xb = wl.float_to_bf16_bits(x)
    xq, xs = lib.rotate_quant(bf16_to_dev(xb))
    xq_ref, xs_ref = oracle.rotate_quant(xb, 256)
    xq = xq.cpu().numpy()
    assert np.all(xq[0] == 0) and xs.cpu().numpy()[0] == 0
    assert np.all(np.abs(xq[1, :256]) == 127)
    assert_scales_close(xs.cpu().numpy(), xs_ref)
    q_exact = exact_quotients(wl.bf16_bits_to_float(xb), xs_ref, 256)
    assert_codes_off_ties(xq, xq_ref, q_exact)


@pytest.mark.parametrize("K", [4096, 4352])
def test_rotate_quant_tiny_rows(lib, K):
    """Rows whose scale is far below 1: normal scales must match exactly as
    for ordinary rows; where the oracle's fp32 scale is subnormal it carries
    fewer bits, so codes may differ by 1 and scales by one subnormal step."""
    say(f"rotate_quant tiny rows K={K}")
    rng = np.random.default_rng(77)
    x = np.zeros((5, K), dtype=np.float32)
    x[0] = 1e-33                                   # constant groups, scale ~1e-35
    x[1] = rng.standard_normal(K) * 1e-32          # random, scale ~1e-35 (normal)
    x[2] = rng.standard_normal(K) * 1e-36          # scale near the subnormal edge
    x[3, ::7] = 2.0 ** -130                        # bf16 subnormal entries
    x[4] = rng.standard_normal(K)                  # an ordinary row beside them
    xb = wl.float_to_bf16_bits(x)
    xq, xs = lib.rotate_quant(bf16_to_dev(xb))
    xq, xs = xq.cpu().numpy(), xs.cpu().numpy()
    xq_ref, xs_ref = oracle.rotate_quant(xb, 256)
    normal = xs_ref >= np.float32(2.0 ** -126)
    assert normal[[0, 1, 4]].all()
    assert_scales_close(xs[normal], xs_ref[normal])
    assert_codes_close(xq[normal], xq_ref[normal])
    assert np.array_equal(xq[0], xq_ref[0])
    sub = ~normal
    assert np.all(np.abs(xs[sub].astype(np.float64) - xs_ref[sub]) <= 2.0 ** -149 * 1.5)
    assert np.abs(xq[sub].astype(np.int16) - xq_ref[sub]).max(initial=0) <= 1
    assert np.all(np.abs(xq).max(axis=1) == 127)


def test_rotate_quant_ties_half_away(lib):
    say("rotate_quant exact ties")
    import scipy.linalg
    v = np.zeros(256)
    v[0], v[1], v[2] = 127.0, 0.5, -0.5
    x = v @ (scipy.linalg.hadamard(256) / 16.0)
    xb = wl.float_to_bf16_bits(x[None, :].astype(np.float32))
    xq, xs = lib.rotate_quant(bf16_to_dev(xb))
    q = xq.cpu().numpy()[0]
    assert xs.cpu().numpy()[0] == 1.0
    assert q[0] == 127 and q[1] == 1 and q[2] == -1 and np.all(q[3:] == 0)


# ----------------------------------------------------- weight preparation

@pytest.mark.parametrize("N,K,g,dtype", [(256, 512, 256, "f32"), (1000, 4096, 256, "f32"),
                                         (300, 4096, 256, "bf16"), (64, 12288, 256, "f32"),
                                         (128, 4096, 16, "f32"), (128, 2048, 1, "f32")])
def test_quantize_weight_i8_parity(lib, N, K, g, dtype):
    import torch
    say(f"quantize_weight i8 N={N} K={K} group={g} {dtype}")
    w = wl.make_weight(N, K, seed=N + K + g)
    if dtype == "bf16":
        wb = wl.float_to_bf16_bits(w)
        w = wl.bf16_bits_to_float(wb)
        wd = bf16_to_dev(wb)
    else:
        wd = to_dev(w)
    wq, ws = lib.quantize_weight(wd, group=g, bits=8)
    wq_ref, ws_ref = oracle.quantize_weight_i8(w, g)
    assert_scales_close(ws.cpu().numpy(), ws_ref)
    assert_codes_close(wq.cpu().numpy(), wq_ref)
    del torch


def _check_i4_rows(w, g, ci, ws, wq4, what):
    """int4 weight prep on the GPU against the oracle: the clip choice is the
    oracle's argmin or a near tie with it (assert_clip_choice), and the
    scales and codes equal the oracle's at the candidate the GPU chose
    (oracle with force_index), to the codes' usual bar."""
    _, _, _, err = oracle.quantize_weight_i4(w, g, with_errors=True)
    rot_norm = np.linalg.norm(oracle.rotate_rows(w.astype(np.float64), g), axis=1)
    off = assert_clip_choice(ci, err, rot_norm, what)
    wq4_at, ws_at, ci_at = oracle.quantize_weight_i4(w, g, force_index=ci)
    assert np.array_equal(ci_at, ci)
    assert_scales_close(ws, ws_at, f"{what}: scales")
    q = oracle.unpack_i4(wq4)
    assert np.abs(q).max(initial=0) <= 7
    assert_codes_close(q, oracle.unpack_i4(wq4_at), f"{what}: int4 codes")
    return off


@pytest.mark.parametrize("N,K,g", [(64, 512, 256), (256, 4096, 256), (32, 12288, 256), (64, 1024, 16)])
def test_quantize_weight_i4_parity(lib, N, K, g):
    say(f"quantize_weight i4 N={N} K={K} group={g}")
    w = wl.make_weight(N, K, seed=5 * N + K + g)
    w[:, :: max(1, K // 7)] *= 25.0  # a few heavy columns so the search has to clip
    wq4, ws, ci = lib.quantize_weight(to_dev(w), group=g, bits=4, with_clip_index=True)
    off = _check_i4_rows(w, g, ci.cpu().numpy(), ws.cpu().numpy(), wq4.cpu().numpy(), f"i4 N={N} K={K}")
    say(f"  rows off the oracle's argmin (near ties): {off}")


@pytest.mark.parametrize("g", [1, 256])
def test_quantize_weight_i4_zero_rows_keep_the_larger_c(lib, g):
    """All-zero rows (every clip candidate has error 0) take the first
    candidate, c = 1.00, as the oracle does; a normal row beside them is
    checked like any other."""
    say(f"quantize_weight i4 zero rows group={g}")
    K = 512
    w = np.zeros((3, K), dtype=np.float32)
    w[1] = wl.make_weight(1, K, seed=77)[0]
    wq4, ws, ci = lib.quantize_weight(to_dev(w), group=g, bits=4, with_clip_index=True)
    ci, ws, wq4 = ci.cpu().numpy(), ws.cpu().numpy(), wq4.cpu().numpy()
    assert ci[0] == 0 and ci[2] == 0
    assert ws[0] == 0 and ws[2] == 0
    q = oracle.unpack_i4(wq4)
    assert not q[0].any() and not q[2].any()
    _check_i4_rows(w, g, ci, ws, wq4, "i4 zero rows")


# -------------------------------------------------------------- end to end

def _linear_full(lib, key):
    cfg = wl.CONFIGS[key]
    x, w = wl.config_inputs(key)
    bits = cfg.wbits
    say(f"{key}: weight prep on GPU (bits={bits})")
    ci = None
    if bits == 8:
        wq, ws = lib.quantize_weight(to_dev(w), bits=8)
        y = lib.w8a8_linear(bf16_to_dev(x), wq, ws)
    else:
        wq, ws, ci = lib.quantize_weight(to_dev(w), bits=4, with_clip_index=True)
        y = lib.w4a8_linear(bf16_to_dev(x), wq, ws)
    return cfg, x, w, wq, ws, y, ci


@pytest.mark.parametrize("key", ["C1", "C2"])
def test_linear_config_full(lib, key):
    cfg, x, w, wq, ws, y, _ = _linear_full(lib, key)
    say(f"{key}: oracle")
    wq_ref, ws_ref = oracle.quantize_weight_i8(w, 256)
    assert_scales_close(ws.cpu().numpy(), ws_ref)
    assert_codes_close(wq.cpu().numpy(), wq_ref, "weight codes")
    xq, xs = lib.rotate_quant(bf16_to_dev(x))
    xq_ref, xs_ref = oracle.rotate_quant(x, 256)
    assert_codes_close(xq.cpu().numpy(), xq_ref, "activation codes")
    y_ref = oracle.w8a8_linear(x, wq_ref, ws_ref, 256)
    r = assert_rel_l2(bf16_from_dev(y), y_ref)
    say(f"{key}: rel L2 {r:.2e}")


def _sampled_check(lib, key, n_tok=64, n_rows=192):
    """Full-size config, GPU output checked on sampled (token, row) pairs that
    the oracle computes from the same inputs."""
    cfg, x, w, wq, ws, y, ci = _linear_full(lib, key)
    M, K = x.shape
    N = w.shape[0]
    rng = np.random.default_rng(99)
    toks = np.sort(rng.choice(M, n_tok, replace=False))
    rows = np.sort(rng.choice(N, n_rows, replace=False))
    say(f"{key}: oracle on {n_tok} tokens x {n_rows} rows")
    xq_ref, xs_ref = oracle.rotate_quant(x[toks], 256)
    if cfg.wbits == 8:
        wq_ref, ws_ref = oracle.quantize_weight_i8(w[rows], 256)
        w_codes_ref = wq_ref
        w_codes = wq.cpu().numpy()[rows]
    else:
        wq4_ref, ws_ref, _ = oracle.quantize_weight_i4(w[rows], 256)
        w_codes_ref = oracle.unpack_i4(wq4_ref)
        w_codes = oracle.unpack_i4(wq.cpu().numpy()[rows])
    y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref, w_codes_ref), xs_ref, ws_ref)
    y_s = bf16_from_dev(y)[np.ix_(toks, rows)]
    r = assert_rel_l2(y_s, y_ref)
    if cfg.wbits == 8:
        assert_codes_close(w_codes, w_codes_ref, "weight codes")
        assert_scales_close(ws.cpu().numpy()[rows], ws_ref, "weight scales")
    else:
        _check_i4_rows(np.ascontiguousarray(w[rows]), 256, ci.cpu().numpy()[rows], ws.cpu().numpy()[rows],
                       wq.cpu().numpy()[rows], f"{key} weight rows")
    xq, _ = lib.rotate_quant(bf16_to_dev(x))
    assert_codes_close(xq.cpu().numpy()[toks], xq_ref, "activation codes")
    say(f"{key}: sampled rel L2 {r:.2e}")


@pytest.mark.parametrize("key", ["C3u", "C3d", "C5"])
def test_linear_config_sampled(lib, key):
    _sampled_check(lib, key)


def test_w4a8_small_full(lib):
    say("w4a8 small full")
    rng = np.random.default_rng(4)
    x = wl.make_activations(48, 1024, 10, seed=41)
    w = wl.make_weight(96, 1024, seed=41)
    wq4, ws = lib.quantize_weight(to_dev(w), bits=4)
    y = lib.w4a8_linear(bf16_to_dev(x), wq4, ws)
    wq4_ref, ws_ref, _ = oracle.quantize_weight_i4(w, 256)
    y_ref = oracle.w4a8_linear(x, wq4_ref, ws_ref, 256)
    assert_rel_l2(bf16_from_dev(y), y_ref)
    del rng


@pytest.mark.parametrize("M,K,N,g", [(1, 256, 16, 256), (33, 4352, 70, 256), (100, 1152, 300, 16),
                                     (5, 2048, 1024, 1), (17, 32768, 64, 256)])
def test_linear_edge_shapes(lib, M, K, N, g):
    say(f"w8a8 edge M={M} K={K} N={N} group={g}")
    x = wl.make_activations(M, K, max(1, K // 100), seed=M + K + N)
    w = wl.make_weight(N, K, seed=M + K + N)
    wq, ws = lib.quantize_weight(to_dev(w), group=g)
    y = lib.w8a8_linear(bf16_to_dev(x), wq, ws, group=g)
    wq_ref, ws_ref = oracle.quantize_weight_i8(w, g)
    y_ref = oracle.w8a8_linear(x, wq_ref, ws_ref, g)
    assert_rel_l2(bf16_from_dev(y), y_ref)


def test_deterministic(lib):
    say("determinism")
    x, w = wl.config_inputs("C2")
    wq, ws = lib.quantize_weight(to_dev(w))
    xd = bf16_to_dev(x)
    y1 = bf16_from_dev(lib.w8a8_linear(xd, wq, ws))
    y2 = bf16_from_dev(lib.w8a8_linear(xd, wq, ws))
    assert np.array_equal(y1, y2)


def test_no_out_of_bounds_writes(lib):
    """Canary-padded buffers: the kernels write exactly their outputs, and a
    rejected call writes nothing."""
    import torch
    say("canaries")
    M, K, N = 37, 512, 70
    x = wl.make_activations(M, K, 5, seed=3)
    w = wl.make_weight(N, K, seed=3)
    wq, ws = lib.quantize_weight(to_dev(w))
    pad = 4096
    ybuf = torch.full((pad + M * N + pad,), 0x7E7E, dtype=torch.int16, device="cuda")
    y = ybuf[pad:pad + M * N].view(M, N).view(torch.bfloat16)
    lib.w8a8_linear(bf16_to_dev(x), wq, ws, out=y)
    yb = ybuf.cpu().numpy()
    assert np.all(yb[:pad] == 0x7E7E) and np.all(yb[pad + M * N:] == 0x7E7E)
    # rejected call (group 3): nothing written
    ybuf.fill_(0x1234)
    ws_bytes = lib.convrot_workspace_size(M, K)
    wsp = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    rc = lib.convrot_w8a8_linear(bf16_to_dev(x), M, K, wq, ws, N, 3, y, wsp, ws_bytes)
    torch.cuda.synchronize()
    assert rc == 3
    assert np.all(ybuf.cpu().numpy() == 0x1234)


def test_stack_config_sampled(lib):
    """The 32-layer decoder linear stack (M = 8704): every one of the 224
    linears runs on the GPU; each is checked on sampled tokens x rows."""
    import torch
    cfg = wl.CONFIGS["C4"]
    say("C4: drawing the four shared activation tensors")
    acts = wl.stack_activations()
    acts_dev = [bf16_to_dev(a) for a in acts]
    rng = np.random.default_rng(123)
    worst = 0.0
    for layer in range(cfg.layers):
        for li, lin in enumerate(cfg.linears):
            seed = wl.C4_WEIGHT_SEED_BASE + layer * 16 + li
            w_dev = wl.make_weight_device(lin.N, lin.K, seed, "cuda")
            wq, ws = lib.quantize_weight(w_dev)
            xin = wl.C4_INPUT_OF[lin.name]
            y = lib.w8a8_linear(acts_dev[xin], wq, ws)
            toks = np.sort(rng.choice(cfg.M, 8, replace=False))
            rows = np.sort(rng.choice(lin.N, 48, replace=False))
            w_rows = w_dev[torch.from_numpy(rows).cuda()].cpu().numpy()
            xq_ref, xs_ref = oracle.rotate_quant(acts[xin][toks], 256)
            wq_ref, ws_ref = oracle.quantize_weight_i8(w_rows, 256)
            y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref, wq_ref), xs_ref, ws_ref)
            y_s = bf16_from_dev(y)[np.ix_(toks, rows)]
            r = assert_rel_l2(y_s, y_ref, f"layer {layer} {lin.name}")
            worst = max(worst, r)
            del w_dev, wq, ws, y
        say(f"C4: layer {layer} ok (worst rel L2 so far {worst:.2e})")


def test_concurrent_host_threads(lib):
    """Two host threads, each on its own stream, launching GEMMs of several
    tile plans at once (first calls included, so the per-kernel occupancy
    memo is filled concurrently): results stay bit-exact."""
    import threading
    import torch
    say("gemm_i8 from two host threads on two streams")
    # plans: 64x128 four-stage, 128x128 persistent, range-checked K, 256x256,
    # 256x192 persistent, eight-wave 256x384
    shapes = [(512, 4096, 512), (2048, 12288, 256), (300, 1000, 1040), (8704, 12288, 256), (2048, 6144, 2048),
              (2048, 12288, 2048)]
    errors = []

    def worker(idx):
        try:
            stream = torch.cuda.Stream()
            rng = np.random.default_rng(500 + idx)
            with torch.cuda.stream(stream):
                for rep in range(3):
                    for (M, N, K) in shapes[idx::2] + shapes[1 - idx::2]:
                        a = rng.integers(-127, 128, (M, K), dtype=np.int8)
                        b = rng.integers(-127, 128, (N, K), dtype=np.int8)
                        xs = np.ones(M, np.float32)
                        ws = np.ones(N, np.float32)
                        acc, _ = lib.gemm_i8(to_dev(a), to_dev(xs), to_dev(b), to_dev(ws), wbits=8, want_y=False)
                        stream.synchronize()
                        rows = rng.choice(M, 8, replace=False)
                        ref = a[rows].astype(np.int64) @ b.astype(np.int64).T
                        if not np.array_equal(acc[rows.tolist()].cpu().numpy(), ref):
                            errors.append((idx, M, N, K, rep))
        except Exception as e:  # reported below
            errors.append((idx, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
