"""GPU parity of the weight-only (dequant) path against the oracle: the
dequantized bf16 weight bit for bit (even log2(group)), the bf16 matmul
within its fp32-accumulation bound, and the composed linear."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_rel_l2, bf16_from_dev, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _f(bits):
    return wl.bf16_bits_to_float(bits).astype(np.float64)


def _ulp_bf16(v):
    """Spacing of bf16 values at |v| (2^(e-7)), for normal magnitudes."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_gemm_bf16_close(y_gpu, y_ref, x_bits, w_bits, rows=None, what="y"):
    """|y_gpu - y_ref| <= one bf16 step at y_ref + the fp32 accumulation bound
    K * 2^-24 * sum_k |x w| (the reference is the exact sum rounded to fp32,
    then to bf16); relative L2 <= 1e-3 over the whole block."""
    xf = _f(x_bits)
    wf = _f(w_bits)
    g = _f(y_gpu)
    r = _f(y_ref)
    K = xf.shape[1]
    bound = _ulp_bf16(r) + K * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T) + 2.0 ** -133
    over = np.abs(g - r) > bound
    assert not over.any(), f"{what}: {over.sum()} outputs beyond the accumulation bound"
    assert_rel_l2(y_gpu, y_ref, what)


@pytest.mark.parametrize("wbits,N,K,g", [
    (8, 64, 512, 256), (8, 300, 4096, 256), (8, 33, 1152, 16), (8, 40, 2048, 64), (8, 17, 4096, 4), (8, 9, 1024, 1),
    (4, 64, 512, 256), (4, 100, 4096, 256), (4, 20, 1152, 16), (8, 5, 32768, 256),
    (8, 7, 768, 256), (4, 3, 256, 256), (8, 12288, 4096, 256),   # partial last workgroup; full size
])
def test_dequantize_bit_exact(lib, wbits, N, K, g):
    say(f"dequantize W{wbits} N={N} K={K} group={g}")
    rng = np.random.default_rng(N + K + g + wbits)
    s = (rng.random(N) * 0.01 + 1e-5).astype(np.float32)
    s[0] = 0.0                                                # an all-zero scale row
    if wbits == 8:
        q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    else:
        q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    got = bf16_from_dev(lib.dequantize_weight(to_dev(q), to_dev(s), K, wbits=wbits, group=g))
    assert np.array_equal(got, oracle.dequantize_weight(q, s, g))


@pytest.mark.parametrize("g", [2, 8, 32, 128])
def test_dequantize_odd_groups_within_one_step(lib, g):
    """Odd log2(group): 1/sqrt(g) adds one fp32 rounding on the GPU, so a
    value may land one bf16 step away, on a small fraction of the weights."""
    say(f"dequantize odd group {g}")
    N, K = 64, 2048
    rng = np.random.default_rng(g)
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s = (rng.random(N) * 0.01 + 1e-5).astype(np.float32)
    got = _f(bf16_from_dev(lib.dequantize_weight(to_dev(q), to_dev(s), K, group=g)))
    ref = _f(oracle.dequantize_weight(q, s, g))
    d = np.abs(got - ref)
    assert np.all(d <= _ulp_bf16(ref) * 1.0001)
    assert np.count_nonzero(d) <= 1e-3 * d.size


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (33, 70, 208), (130, 257, 272), (64, 512, 4096), (7, 1024, 12288),
                                   (64, 512, 1088)])
def test_gemm_bf16_full(lib, M, N, K):
    say(f"gemm_bf16 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    x = wl.float_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.float_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    y = bf16_from_dev(lib.gemm_bf16(bf16_to_dev(x), bf16_to_dev(w)))
    assert_gemm_bf16_close(y, oracle.gemm_bf16(x, w), x, w)


@pytest.mark.parametrize("M,N,K", [(2048, 6144, 1024), (8704, 4096, 256), (2000, 12280, 1040), (4096, 12288, 256),
                                   (2048, 4096, 6144), (1990, 4090, 2064), (1000, 4000, 1040), (2048, 4096, 1088)])
def test_gemm_bf16_large_sampled(lib, M, N, K):
    """The large tile plans (persistent 256x192, even and ragged; 256x256;
    128x128 persistent) and the deeper pipelines (256x128 three-stage, even
    and ragged; 128x128 four-stage) on sampled rows against the oracle."""
    say(f"gemm_bf16 large M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K + 1)
    x = wl.float_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.float_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    y = lib.gemm_bf16(bf16_to_dev(x), bf16_to_dev(w))
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), [0, 255, 256, M - 1]]))
    assert_gemm_bf16_close(bf16_from_dev(y[rows.tolist()]), oracle.gemm_bf16(x[rows], w), x[rows], w)


@pytest.mark.parametrize("wbits", [8, 4])
def test_dequant_linear_c3u_sampled(lib, wbits):
    """The weight-only linear at the headline shape (M=2048, K=4096,
    N=12288): the dequantized weight bit-exact, outputs on sampled tokens
    within the bf16 matmul's bound."""
    import torch
    x, w = wl.config_inputs("C3u")
    say(f"dequant_linear W{wbits} C3u")
    wq, ws = lib.quantize_weight(torch.from_numpy(w).cuda(), bits=wbits)
    y = lib.dequant_linear(bf16_to_dev(x), wq, ws, wbits=wbits)
    w_hat = oracle.dequantize_weight(wq.cpu().numpy().view(np.uint8 if wbits == 4 else np.int8), ws.cpu().numpy())
    assert np.array_equal(bf16_from_dev(lib.dequantize_weight(wq, ws, 4096, wbits=wbits)), w_hat)
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(x.shape[0], 12, replace=False))
    assert_gemm_bf16_close(bf16_from_dev(y[toks.tolist()]), oracle.gemm_bf16(x[toks], w_hat), x[toks], w_hat)


def test_dequant_path_is_closer_to_full_precision(lib):
    """Against the full-precision product x . W^T, the weight-only path (bf16
    activations kept) is at least as accurate as W8A8 (activations
    quantized) on the outlier-heavy inputs."""
    import torch
    x, w = wl.config_inputs("C2")
    wq, ws = lib.quantize_weight(torch.from_numpy(w).cuda())
    xd = bf16_to_dev(x)
    y_dq = _f(bf16_from_dev(lib.dequant_linear(xd, wq, ws)))
    y_8 = _f(bf16_from_dev(lib.w8a8_linear(xd, wq, ws)))
    ref = _f(x) @ w.astype(np.float64).T
    e_dq = np.linalg.norm(y_dq - ref) / np.linalg.norm(ref)
    e_8 = np.linalg.norm(y_8 - ref) / np.linalg.norm(ref)
    say(f"rel L2 vs full precision: dequant {e_dq:.3e}, w8a8 {e_8:.3e}")
    assert e_dq <= e_8


@pytest.mark.parametrize("M,N,K", [(4100, 12288, 528), (3000, 7000, 1504), (2000, 4000, 3008), (300, 3000, 2000),
                                   (1000, 4000, 1008), (3000, 3000, 608), (1920, 12288, 1024), (1800, 12288, 2048),
                                   (6000, 12288, 1024), (8704, 12288, 1024)])
def test_gemm_bf16_irregular_guarded(lib, M, N, K):
    """Irregular shapes on every tile plan of the bf16 matmul (256x256,
    256x192, 256x128 three-stage, 64x128 and 128x128 four-stage, 128x128,
    and the eight-wave 256x384 tiles: one round and three whole rounds with
    ragged M, and on the first 8192 of 8704 rows with the ordinary plan on
    the rest):
    sampled rows within the accumulation bound of the oracle, and guard
    words around the output untouched."""
    import torch
    say(f"gemm_bf16 irregular M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 2 * N + 3 * K)
    x = wl.float_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.float_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    guard = 64
    buf = torch.full((guard + M * N + guard,), 0x1234, dtype=torch.int16, device="cuda")
    y = buf[guard:guard + M * N]
    rc = lib.convrot_gemm_bf16(bf16_to_dev(x), bf16_to_dev(w), M, N, K, y)
    torch.cuda.synchronize()
    assert rc == 0
    h = buf.cpu().numpy()
    assert np.all(h[:guard] == 0x1234) and np.all(h[guard + M * N:] == 0x1234)
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), [0, M - 1]]))
    got = h[guard:guard + M * N].reshape(M, N)[rows].view(np.uint16)
    assert_gemm_bf16_close(got, oracle.gemm_bf16(x[rows], w), x[rows], w)
