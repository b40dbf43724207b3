"""GPU parity of the multi-output calls (several weight matrices sharing one
quantized input; one GEMM launch, or one per output where every output
takes the eight-wave tiles) against the oracle and against the
single-output calls, through the C ABI."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_rel_l2, bf16_from_dev, bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _codes(rng, M, K):
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    xs = (rng.random(M) * 0.1 + 1e-3).astype(np.float32)
    return a, xs


def _weights(rng, Ns, K, wbits):
    out = []
    for n in Ns:
        ws = (rng.random(n) * 1e-3 + 1e-5).astype(np.float32)
        if wbits == 8:
            b = rng.integers(-127, 128, (n, K), dtype=np.int8)
            out.append((b, b, ws))
        else:
            packed = rng.integers(0, 256, (n, K // 2), dtype=np.uint8)
            out.append((packed, oracle.unpack_i4(packed), ws))
    return out


@pytest.mark.parametrize("wbits,M,K,Ns", [
    (8, 33, 512, (512, 128, 128)),            # q/k/v-like, small M: 64x128 tiles, four stages
    (8, 130, 272, (70, 257, 33)),             # ragged N and K (tail kernel)
    (8, 300, 1024, (16,) * 8),                # eight tiny outputs
    (8, 2048, 512, (4096, 1024, 1024)),       # 128x128 tiles across three outputs (short K)
    (8, 2048, 256, (12288, 12288)),           # 256x256 tiles (every N a multiple of 256)
    (8, 2048, 2048, (2048, 1024, 1024)),      # 256x128 tiles, three stages, one per CU
    (8, 2048, 2048, (12288, 12288)),          # every output on eight-wave 256x384 tiles, one launch each
    (8, 8704, 2048, (12288, 12288)),          # each output: eight-wave tiles on 8192 rows, then the last 512
    (8, 2048, 2048, (12288, 4096)),           # one output cannot take eight-wave tiles: one multi launch
    (4, 64, 1024, (512, 96, 1000)),           # packed int4
    (4, 4096, 256, (6144, 6144)),             # packed int4, 256x256
])
def test_gemm_multi_bit_exact(lib, wbits, M, K, Ns):
    say(f"gemm_i8_multi W{wbits} M={M} K={K} N={Ns}")
    rng = np.random.default_rng(M + K + sum(Ns) + wbits)
    a, xs = _codes(rng, M, K)
    ws = _weights(rng, Ns, K, wbits)
    res = lib.gemm_i8_multi(to_dev(a), to_dev(xs), [(to_dev(dev), to_dev(s)) for dev, _, s in ws], wbits=wbits)
    rows = np.arange(M) if M <= 300 else np.unique(np.concatenate([rng.choice(M, 48, replace=False), [0, M - 1]]))
    for (acc, y), (_, b, s) in zip(res, ws):
        ref = a[rows].astype(np.int64) @ b.astype(np.int64).T
        assert np.array_equal(acc[rows.tolist()].cpu().numpy(), ref)
        assert np.array_equal(bf16_from_dev(y[rows.tolist()]), oracle.epilogue(ref.astype(np.int32), xs[rows], s))


@pytest.mark.parametrize("wbits", [8, 4])
def test_linear_multi_equals_single_calls(lib, wbits):
    """Decoder q/k/v shapes at M = 8704: each output of the multi call is bit
    for bit the single call's output for the same weight; sampled outputs
    against the oracle."""
    import torch
    M, K, Ns = 8704, 4096, (4096, 1024, 1024)
    say(f"linear_multi W{wbits} M={M} K={K} N={Ns}")
    x = wl.make_activations(M, K, K // 100, seed=41)
    xd = bf16_to_dev(x)
    weights, hosts = [], []
    for i, n in enumerate(Ns):
        w = wl.make_weight(n, K, seed=50 + i)
        wq, wsc = lib.quantize_weight(torch.from_numpy(w).cuda(), bits=wbits)
        weights.append((wq, wsc))
        hosts.append(w)
    ys = lib.linear_multi(xd, weights, wbits=wbits)
    single = lib.w8a8_linear if wbits == 8 else lib.w4a8_linear
    for (wq, wsc), y in zip(weights, ys):
        assert torch.equal(y.view(torch.int16), single(xd, wq, wsc).view(torch.int16))
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(M, 16, replace=False))
    xq_ref, xs_ref = oracle.rotate_quant(x[toks], 256)
    for (wq, wsc), y, w in zip(weights, ys, hosts):
        rows = np.sort(rng.choice(w.shape[0], 64, replace=False))
        if wbits == 8:
            wq_ref, ws_ref = oracle.quantize_weight_i8(w[rows], 256)
        else:
            packed, ws_ref, _ = oracle.quantize_weight_i4(w[rows], 256)
            wq_ref = oracle.unpack_i4(packed)
        y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref, wq_ref), xs_ref, ws_ref)
        assert_rel_l2(bf16_from_dev(y)[np.ix_(toks, rows)], y_ref)


def test_multi_fused_norm_chain(lib):
    """RMSNorm + rotate-quantize once, then the three projections in one
    GEMM launch: equals the oracle's norm, quantize and product per output."""
    M, K, Ns = 96, 2048, (2048, 512, 512)
    say(f"rmsnorm_rotate_quant + gemm_i8_multi M={M} K={K} N={Ns}")
    x = wl.make_activations(M, K, K // 100, seed=60)
    nw = wl.make_norm_weight(K, K // 100, seed=60)
    xq, xs = lib.rmsnorm_rotate_quant(bf16_to_dev(x), to_dev(nw))
    rng = np.random.default_rng(61)
    ws = _weights(rng, Ns, K, 8)
    res = lib.gemm_i8_multi(xq, xs, [(to_dev(b), to_dev(s)) for b, _, s in ws], want_acc=False)
    xq_ref, xs_ref, _ = oracle.rmsnorm_rotate_quant(x, nw)
    for (_, y), (_, b, s) in zip(res, ws):
        y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref, b), xs_ref, s)
        assert_rel_l2(bf16_from_dev(y), y_ref)


def test_multi_no_out_of_bounds_writes(lib):
    """Outputs of ragged N placed back to back in one buffer with guard
    words between them: nothing outside each output is written."""
    import torch
    M, K, Ns = 70, 256, (100, 36, 260)
    say(f"gemm_i8_multi guards M={M} N={Ns}")
    rng = np.random.default_rng(3)
    a, xs = _codes(rng, M, K)
    ws = _weights(rng, Ns, K, 8)
    guard = 64
    sizes = [M * n for n in Ns]
    offs, pos = [], guard
    for sz in sizes:
        offs.append(pos)
        pos += (sz + guard + 7) // 8 * 8
    buf = torch.full((pos + guard,), 0x1234, dtype=torch.int16, device="cuda")
    desc = []
    for (b, _, s), n, off in zip(ws, Ns, offs):
        desc.append((to_dev(b), to_dev(s), n, None, buf[off:off + M * n]))
    rc = lib.convrot_gemm_i8_multi(to_dev(a), to_dev(xs), 8, M, K, desc)
    torch.cuda.synchronize()
    assert rc == 0
    h = buf.cpu().numpy().view(np.uint16)
    mask = np.ones(h.size, dtype=bool)
    for (b, _, s), n, off in zip(ws, Ns, offs):
        mask[off:off + M * n] = False
        y = h[off:off + M * n].reshape(M, n)
        assert np.array_equal(y, oracle.epilogue(oracle.gemm_i8(a, b), xs, s))
    assert np.all(h[mask] == 0x1234)
