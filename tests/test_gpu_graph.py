"""The linear calls inside a captured HIP graph (through torch.cuda.graph):
the library enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so a captured call replays to the eager
result. Each graph is replayed several times with other eager work and
synchronisations between the replays, and every replay is compared bit for
bit with the eager output."""
import numpy as np
import pytest

from tests.gpu_helpers import bf16_to_dev, say, to_dev
from w8a8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


# Headline shape (eight-wave 256x384 tiles), a small one (64x128 tiles,
# four stages), a long-K one (256x128 tiles, three stages), and the decoder
# stack's gate/up shape, whose GEMM is two launches (eight-wave tiles on the
# first 8192 rows, the ordinary plan on the last 512).
@pytest.mark.parametrize("M,K,N", [(2048, 4096, 12288), (512, 4096, 4096), (2048, 12288, 4096),
                                   (8704, 2048, 12288)])
def test_w8a8_linear_graph_replays(lib, M, K, N):
    import torch
    say(f"w8a8_linear in a HIP graph M={M} K={K} N={N}")
    x = bf16_to_dev(wl.make_activations(M, K, K // 100, seed=M + K))
    x2 = bf16_to_dev(wl.make_activations(M, K, K // 100, seed=M + K + 1))
    wq, ws = lib.quantize_weight(to_dev(wl.make_weight(N, K, seed=N)))
    y_eager = lib.w8a8_linear(x, wq, ws)
    y2_eager = lib.w8a8_linear(x2, wq, ws)
    out = torch.empty_like(y_eager)
    wsp = lib.workspace(M, K)
    lib.w8a8_linear(x, wq, ws, out=out, ws=wsp)  # first call outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.w8a8_linear(x, wq, ws, out=out, ws=wsp)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        # eager work on the same buffers between replays
        y2 = lib.w8a8_linear(x2, wq, ws, out=torch.empty_like(y_eager), ws=wsp)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y2_eager.view(torch.int16))


def test_linear_multi_graph_replays(lib):
    """Fused RMSNorm + rotate-quantize, then three projections in one GEMM
    launch, captured together."""
    import torch
    M, K, Ns = 1024, 2048, (2048, 512, 512)
    say(f"rmsnorm + gemm_i8_multi in a HIP graph M={M} K={K} N={Ns}")
    x = bf16_to_dev(wl.make_activations(M, K, K // 100, seed=5))
    nw = to_dev(wl.make_norm_weight(K, K // 100, seed=5))
    weights = [lib.quantize_weight(to_dev(wl.make_weight(n, K, seed=60 + i))) for i, n in enumerate(Ns)]

    def run():
        xq, xs = lib.rmsnorm_rotate_quant(x, nw)
        return [y for _, y in lib.gemm_i8_multi(xq, xs, weights, want_acc=False)]

    eager = run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = run()
    for rep in range(3):
        for y in captured:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, ye in zip(captured, eager):
            assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), f"replay {rep}"
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_rmsnorm_token_walk_graph_replays(lib):
    """The fused norm call without the bf16 output at 4100 tokens, K 4096
    (the workgroups walk the tokens on the resident grid), captured alone:
    codes and scales of every replay equal the eager call's."""
    import torch
    M, K = 4100, 4096
    say(f"rmsnorm_rotate_quant (token walk) in a HIP graph M={M} K={K}")
    x = bf16_to_dev(wl.make_activations(M, K, K // 100, seed=11))
    nw = to_dev(wl.make_norm_weight(K, K // 100, seed=11))
    q_eager, s_eager = lib.rmsnorm_rotate_quant(x, nw)
    q = torch.empty_like(q_eager)
    s = torch.empty_like(s_eager)
    rc = lib.convrot_rmsnorm_rotate_quant(x, nw, 1e-6, M, K, 256, q, s, None)  # first call outside the capture
    assert rc == 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.convrot_rmsnorm_rotate_quant(x, nw, 1e-6, M, K, 256, q, s, None)
    for rep in range(3):
        q.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_eager), f"replay {rep}"
        assert torch.equal(s, s_eager), f"replay {rep}"
        lib.rmsnorm_rotate_quant(x, nw)  # eager work between replays
        torch.cuda.synchronize()
