"""GEMM on irregular shapes (drawn once with a fixed seed, then written out
here), two or three per tile plan, int8 and packed int4 weights: int32
accumulators bit-exact and bf16 outputs bit-exact against the oracle's
epilogue on sampled rows, and guard words around both output buffers
untouched (no write outside [M, N])."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

# (wbits, M, N, K) and the tile plan the shape takes on a 256-CU MI355X.
SHAPES = [
    (8, 6000, 8448, 1040),    # 256x256
    (4, 4100, 12288, 2080),   # 256x256, packed int4
    (8, 4211, 3840, 5904),    # 256x192
    (8, 8704, 4096, 2048),    # 256x256 on rows 0..8191 (two rounds), the last 512 rows on the ordinary plan
    (8, 8700, 4096, 2048),    # the same with 508 ragged rows after the two rounds
    (4, 3973, 6684, 3136),    # 256x192, packed int4
    (4, 1806, 4864, 5088),    # 256x192, packed int4
    (8, 1916, 3894, 7504),    # 256x128, three stages
    (8, 1034, 5888, 2560),    # 256x128, three stages
    (8, 2951, 2180, 6432),    # 256x128, three stages
    (4, 2027, 722, 2464),     # 64x128, four stages, packed int4
    (4, 48, 6497, 6752),      # 64x128, four stages, packed int4
    (8, 69, 8733, 4080),      # 64x128, four stages
    (8, 4971, 640, 1488),     # 128x128, four stages
    (4, 8733, 186, 4000),     # 128x128, four stages, packed int4
    (4, 1204, 2496, 5440),    # 128x128, four stages, packed int4
    (4, 3069, 10752, 1344),   # 128x128, packed int4
    (4, 5384, 1407, 512),     # 128x128, packed int4
    (8, 1357, 5632, 448),     # 128x128
    (8, 2048, 12288, 4096),   # 256x384, eight waves: one round
    (8, 1920, 12288, 2048),   # 256x384, eight waves: one round, ragged M
    (8, 4000, 12288, 4096),   # 256x384, eight waves: two rounds, ragged M
    (8, 1024, 24576, 2048),   # 256x384, eight waves
    (8, 6000, 12288, 2048),   # 256x384, eight waves: three whole rounds, ragged M
    (8, 8704, 12288, 2048),   # 256x384 on rows 0..8191 (four rounds), the last 512 rows on the ordinary plan
    (8, 7000, 12288, 2048),   # 256x384 on rows 0..6143 (three rounds), 856 ragged rows on the ordinary plan
    (4, 2048, 12288, 4096),   # 256x192, packed int4
    (4, 3900, 12288, 2048),   # 256x256, packed int4, ragged M
]
GUARD = 64  # elements before and after each output


@pytest.mark.parametrize("wbits,M,N,K", SHAPES)
def test_gemm_irregular_shapes(lib, wbits, M, N, K):
    import torch
    say(f"gemm_i8 W{wbits} irregular M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K + wbits)
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
    ybuf = torch.full((GUARD + M * N + GUARD,), 0x1234, dtype=torch.int16, device="cuda")
    abuf = torch.full((GUARD + M * N + GUARD,), 0x5a5a5a5a, dtype=torch.int32, device="cuda")
    y, acc = ybuf[GUARD:GUARD + M * N], abuf[GUARD:GUARD + M * N]
    rc = lib.convrot_gemm_i8(to_dev(a), to_dev(xs), wdev, wbits, to_dev(ws), M, N, K, acc, y)
    torch.cuda.synchronize()
    assert rc == 0
    yh = ybuf.cpu().numpy()
    ah = abuf.cpu().numpy()
    assert np.all(yh[:GUARD] == 0x1234) and np.all(yh[GUARD + M * N:] == 0x1234)
    assert np.all(ah[:GUARD] == 0x5a5a5a5a) and np.all(ah[GUARD + M * N:] == 0x5a5a5a5a)
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 32), replace=False), [0, M - 1]]))
    # exact in float64: every partial sum is an integer below 2^53
    ref = np.rint(a[rows].astype(np.float64) @ b.astype(np.float64).T).astype(np.int64)
    got = ah[GUARD:GUARD + M * N].reshape(M, N)[rows]
    assert np.array_equal(got, ref)
    yref = oracle.epilogue(ref.astype(np.int32), xs[rows], ws)
    assert np.array_equal(yh[GUARD:GUARD + M * N].reshape(M, N)[rows].view(np.uint16), yref)


@pytest.mark.parametrize("M,N,K", [(1920, 12288, 2048), (2048, 12288, 4096), (8704, 12288, 2048)])
def test_gemm_eight_wave_single_outputs(lib, M, N, K):
    """The eight-wave 256x384 plan (at M 8704: on the first 8192 rows, the
    ordinary plan on the rest) asked for the int32 accumulators alone and
    for the bf16 output alone: each equal to the same call with both."""
    import torch
    say(f"gemm_i8 eight-wave single outputs M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    a = to_dev(rng.integers(-127, 128, (M, K), dtype=np.int8))
    b = to_dev(rng.integers(-127, 128, (N, K), dtype=np.int8))
    xs = to_dev((rng.random(M) * 0.1 + 1e-3).astype(np.float32))
    ws = to_dev((rng.random(N) * 1e-3 + 1e-5).astype(np.float32))
    acc_both = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y_both = torch.empty((M, N), dtype=torch.int16, device="cuda")
    acc_only = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
    y_only = torch.full((M, N), 7, dtype=torch.int16, device="cuda")
    assert lib.convrot_gemm_i8(a, xs, b, 8, ws, M, N, K, acc_both, y_both) == 0
    assert lib.convrot_gemm_i8(a, xs, b, 8, ws, M, N, K, acc_only, None) == 0
    assert lib.convrot_gemm_i8(a, xs, b, 8, ws, M, N, K, None, y_only) == 0
    torch.cuda.synchronize()
    assert torch.equal(acc_only, acc_both)
    assert torch.equal(y_only, y_both)


@pytest.mark.parametrize("M,N,K", [(2048, 12288, 2048), (8704, 12288, 2048)])
def test_gemm_eight_wave_accumulators_without_scales(lib, M, N, K):
    """The eight-wave plan (one round; and on the first 8192 of 8704 rows)
    asked for the int32 accumulators alone with no scales at all (null
    pointers, which the call allows when it writes no bf16 output): the same
    accumulators as a call that passes scales."""
    import torch
    say(f"gemm_i8 eight-wave accumulators without scales M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 2 * N + K)
    a = to_dev(rng.integers(-127, 128, (M, K), dtype=np.int8))
    b = to_dev(rng.integers(-127, 128, (N, K), dtype=np.int8))
    xs = to_dev((rng.random(M) * 0.1 + 1e-3).astype(np.float32))
    ws = to_dev((rng.random(N) * 1e-3 + 1e-5).astype(np.float32))
    acc_ref = torch.empty((M, N), dtype=torch.int32, device="cuda")
    acc = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
    assert lib.convrot_gemm_i8(a, xs, b, 8, ws, M, N, K, acc_ref, None) == 0
    assert lib.convrot_gemm_i8(a, None, b, 8, None, M, N, K, acc, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(acc, acc_ref)
