"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

- every function include/convrot.h declares is exported by libconvrot.so and
  bound by the Python module;
- argument validation returns the documented status before any device work
  (only invalid argument sets are passed, so nothing is ever enqueued).
"""
import ctypes
import os
import re

import pytest

import w8a8_quantized_linear_amd as cr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cr.library_path()):
        pytest.skip("libconvrot.so not built (run __graft_entry__.build())")
    return cr.load()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("convrot_quantize_weight", "convrot_rotate_quant", "convrot_w8a8_linear", "convrot_w4a8_linear"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in convrot.h but not exported"
    assert sorted(cr.exported_symbols()) == declared_functions()


def test_library_reads_no_environment():
    """The library as built takes no settings from the environment: the
    tile-forcing overrides exist only in tuning builds (-DCONVROT_TUNING)."""
    import shutil
    import subprocess
    lib = cr.library_path()
    if not os.path.exists(lib):
        pytest.skip("libconvrot.so not built (run __graft_entry__.build())")
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert not imported & {"getenv", "secure_getenv"}, "the library reads environment variables"


def test_status_strings_and_version(L):
    for s in range(0, 10):
        assert len(cr.convrot_status_string(s)) > 0
    assert "unknown" in cr.convrot_status_string(99)
    assert cr.convrot_version() >= 100


def test_workspace_size(L):
    assert cr.convrot_workspace_size(0, 4096) == 0
    assert cr.convrot_workspace_size(2048, 4096) == 2048 * 4096 + 2048 * 4
    ws = cr.convrot_workspace_size(3, 16)
    assert ws == 256 + 256 and ws % 256 == 0


# Fake device addresses: non-NULL and 16-byte aligned.  Every call below
# fails validation, so they are never dereferenced.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
D = ctypes.c_void_p(0x40000)
E = ctypes.c_void_p(0x50000)
MIS = ctypes.c_void_p(0x10008)
NUL = None
S0 = ctypes.c_void_p(0)

ERR = {"null": 1, "shape": 2, "group": 3, "align": 4, "ws": 5, "dtype": 7, "arg": 8, "scratch": 9}


def rq(x, M, K, g, q, s):
    return cr.load().convrot_rotate_quant(x, M, K, g, q, s, S0)


def nrq(x, w, eps, M, K, g, q, s, y):
    return cr.load().convrot_rmsnorm_rotate_quant(x, w, eps, M, K, g, q, s, y, S0)


def lin8(x, M, K, w, ws, N, g, y, wsp, wsb):
    return cr.load().convrot_w8a8_linear(x, M, K, w, ws, N, g, y, wsp, wsb, S0)


def lin4(x, M, K, w, ws, N, g, y, wsp, wsb):
    return cr.load().convrot_w4a8_linear(x, M, K, w, ws, N, g, y, wsp, wsb, S0)


def qw(w, dt, N, K, g, bits, q, s):
    return cr.load().convrot_quantize_weight(w, dt, N, K, g, bits, q, s, S0)


def gemm(xq, xs, wq, wb, wsc, M, N, K, acc, y):
    return cr.load().convrot_gemm_i8(xq, xs, wq, wb, wsc, M, N, K, acc, y, S0)


def test_rotate_quant_validation(L):
    assert rq(NUL, 4, 256, 256, B, C) == ERR["null"]
    assert rq(A, 4, 256, 256, NUL, C) == ERR["null"]
    assert rq(A, 4, 300, 256, B, C) == ERR["shape"]       # K % 16
    assert rq(A, 4, 272, 256, B, C) == ERR["shape"]       # K % group
    assert rq(A, 4, 65536, 256, B, C) == ERR["shape"]     # K too large
    assert rq(A, -1, 256, 256, B, C) == ERR["shape"]
    assert rq(A, 4, 256, 3, B, C) == ERR["group"]
    assert rq(A, 4, 512, 512, B, C) == ERR["group"]
    assert rq(A, 4, 256, 0, B, C) == ERR["group"]
    assert rq(MIS, 4, 256, 256, B, C) == ERR["align"]
    assert rq(A, 4, 256, 256, MIS, C) == ERR["align"]
    assert rq(A, 4, 256, 256, B, ctypes.c_void_p(0x30002)) == ERR["align"]
    assert rq(NUL, 0, 256, 256, NUL, NUL) == 0             # empty input: no-op


def test_rmsnorm_rotate_quant_validation(L):
    W4 = ctypes.c_void_p(0x60000)
    assert nrq(NUL, W4, 1e-6, 4, 256, 256, B, C, D) == ERR["null"]
    assert nrq(A, NUL, 1e-6, 4, 256, 256, B, C, D) == ERR["null"]
    assert nrq(A, W4, 1e-6, 4, 256, 256, NUL, C, D) == ERR["null"]
    assert nrq(A, W4, 1e-6, 4, 256, 256, B, NUL, D) == ERR["null"]
    assert nrq(A, W4, -1e-6, 4, 256, 256, B, C, D) == ERR["arg"]
    assert nrq(A, W4, float("nan"), 4, 256, 256, B, C, D) == ERR["arg"]
    assert nrq(A, W4, float("inf"), 4, 256, 256, B, C, D) == ERR["arg"]
    assert nrq(A, W4, 1e-6, 4, 300, 256, B, C, D) == ERR["shape"]
    assert nrq(A, W4, 1e-6, 4, 272, 256, B, C, D) == ERR["shape"]
    assert nrq(A, W4, 1e-6, -1, 256, 256, B, C, D) == ERR["shape"]
    assert nrq(A, W4, 1e-6, 4, 256, 48, B, C, D) == ERR["group"]
    assert nrq(A, ctypes.c_void_p(0x60004), 1e-6, 4, 256, 256, B, C, D) == ERR["align"]   # norm_w: 16 bytes
    assert nrq(A, W4, 1e-6, 4, 256, 256, B, C, MIS) == ERR["align"]
    assert nrq(MIS, W4, 1e-6, 4, 256, 256, B, C, NUL) == ERR["align"]
    assert nrq(NUL, NUL, 1e-6, 0, 256, 256, NUL, NUL, NUL) == 0   # empty input: no-op


def test_linear_validation(L):
    need = cr.convrot_workspace_size(8, 512)
    assert lin8(A, 8, 512, B, C, 64, 256, D, E, need - 1) == ERR["ws"]
    assert lin8(A, 8, 512, B, C, 64, 256, D, NUL, need) == ERR["null"]
    assert lin8(A, 8, 512, B, C, 0, 256, D, E, need) == ERR["shape"]
    assert lin8(A, 8, 500, B, C, 64, 256, D, E, need) == ERR["shape"]
    assert lin8(A, 8, 512, B, C, 64, 256, MIS, E, need) == ERR["align"]
    assert lin8(A, 8, 512, B, C, 64, 256, D, MIS, need) == ERR["align"]
    assert lin8(A, 8, 512, B, C, 64, 100, D, E, need) == ERR["group"]
    assert lin4(A, 8, 528, B, C, 64, 16, D, E, need) == ERR["shape"]   # int4 needs K % 32
    assert lin8(NUL, 0, 512, NUL, NUL, 64, 256, NUL, NUL, 0) == 0
    # N <= 0 is a shape error for every call that multiplies, even with M == 0
    assert lin8(NUL, 0, 512, NUL, NUL, 0, 256, NUL, NUL, 0) == ERR["shape"]
    assert lin4(NUL, 0, 512, NUL, NUL, 0, 256, NUL, NUL, 0) == ERR["shape"]
    assert gemm(NUL, NUL, NUL, 8, NUL, 0, 0, 64, NUL, NUL) == ERR["shape"]
    assert lin8(A, 1 << 31, 512, B, C, 64, 256, D, E, need) == ERR["shape"]


def test_quantize_weight_validation(L):
    assert qw(A, 2, 8, 256, 256, 8, B, C) == ERR["dtype"]
    assert qw(A, 0, 8, 256, 256, 5, B, C) == ERR["dtype"]
    assert qw(A, 0, 8, 250, 256, 8, B, C) == ERR["shape"]
    assert qw(A, 0, 8, 272, 16, 4, B, C) == ERR["shape"]   # int4, K % 32
    assert qw(A, 0, -1, 256, 256, 8, B, C) == ERR["shape"]
    assert qw(NUL, 0, 8, 256, 256, 8, B, C) == ERR["null"]
    assert qw(A, 0, 8, 256, 256, 8, MIS, C) == ERR["align"]
    assert qw(NUL, 0, 0, 256, 256, 8, NUL, NUL) == 0


def test_gemm_validation(L):
    assert gemm(A, B, C, 8, D, 4, 4, 64, NUL, NUL) == ERR["null"]     # no output requested
    assert gemm(A, NUL, C, 8, D, 4, 4, 64, NUL, E) == ERR["null"]     # y needs scales
    assert gemm(A, B, C, 3, D, 4, 4, 64, E, NUL) == ERR["dtype"]
    assert gemm(A, B, C, 8, D, 4, 0, 64, E, NUL) == ERR["shape"]
    assert gemm(A, B, C, 4, D, 4, 4, 48, E, NUL) == ERR["shape"]
    assert gemm(A, B, C, 8, D, 4, 4, 64, MIS, NUL) == ERR["align"]
    assert gemm(NUL, NUL, NUL, 8, NUL, 0, 4, 64, NUL, NUL) == 0
    big = (1 << 30) + 1                                              # 32-bit tile indexing bound
    assert gemm(A, B, C, 8, D, big, 4, 64, E, NUL) == ERR["shape"]
    assert gemm(A, B, C, 8, D, 4, big, 64, E, NUL) == ERR["shape"]


def outs_arr(*rows):
    arr = (cr.LinearOut * len(rows))()
    for i, r in enumerate(rows):
        arr[i] = cr.LinearOut(*r)
    return arr


def gm(xq, xs, wb, M, K, outs, n=None):
    return cr.load().convrot_gemm_i8_multi(xq, xs, wb, M, K, outs, len(outs) if n is None else n, S0)


def lm(x, M, K, g, wb, outs, wsp, wsb, n=None):
    return cr.load().convrot_linear_multi(x, M, K, g, wb, outs, len(outs) if n is None else n, wsp, wsb, S0)


def test_multi_validation(L):
    ok = (0x100000, 0x200000, 512, 0x300000, 0x400000)       # wq, w_scale, N, acc_out, y
    ok_y = (0x500000, 0x600000, 128, None, 0x700000)
    assert gm(A, B, 8, 4, 64, outs_arr(ok), n=0) == ERR["arg"]
    assert gm(A, B, 8, 4, 64, outs_arr(*[ok] * 9)) == ERR["arg"]
    assert gm(A, B, 3, 4, 64, outs_arr(ok)) == ERR["dtype"]
    assert gm(A, B, 8, 4, 48 + 1, outs_arr(ok)) == ERR["shape"]
    assert gm(A, B, 4, 4, 48, outs_arr(ok)) == ERR["shape"]          # int4 needs K % 32
    assert gm(A, B, 8, 4, 64, outs_arr(ok, (0x100000, 0x200000, 0, 0x300000, 0x400000))) == ERR["shape"]
    assert gm(A, B, 8, 4, 64, outs_arr(ok, (0x100000, 0x200000, (1 << 30) + 1, 0x300000, 0x400000))) == ERR["shape"]
    assert gm(A, B, 8, 4, 64, outs_arr(ok, ok_y)) == ERR["null"]     # acc_out in one output only
    assert gm(A, B, 8, 4, 64, outs_arr((0x100000, 0x200000, 64, None, None))) == ERR["null"]
    assert gm(A, B, 8, 4, 64, outs_arr((0x100000, None, 64, 0x300000, 0x400000))) == ERR["null"]  # y needs w_scale
    assert gm(A, NUL, 8, 4, 64, outs_arr(ok)) == ERR["null"]         # y needs x_scale
    assert gm(A, B, 8, 4, 64, outs_arr((0x100008, 0x200000, 64, 0x300000, 0x400000))) == ERR["align"]
    assert gm(A, B, 8, 4, 64, outs_arr((0x100000, 0x200002, 64, 0x300000, 0x400000))) == ERR["align"]
    assert gm(MIS, B, 8, 4, 64, outs_arr(ok)) == ERR["align"]
    assert gm(NUL, NUL, 8, 0, 64, outs_arr(ok)) == 0                   # empty input: no-op
    assert cr.load().convrot_gemm_i8_multi(A, B, 8, 4, 64, None, 1, S0) == ERR["null"]
    # 128-row tiles of all outputs must stay below 2^31
    big = (0x100000, 0x200000, 1 << 30, 0x300000, 0x400000)
    assert gm(A, B, 8, 1 << 30, 64, outs_arr(big)) == ERR["shape"]
    need = cr.convrot_workspace_size(8, 512)
    assert lm(A, 8, 512, 256, 8, outs_arr(ok_y), E, need - 1) == ERR["ws"]
    assert lm(A, 8, 512, 256, 8, outs_arr((0x100000, 0x200000, 64, 0x300000, None)), E, need) == ERR["null"]
    assert lm(A, 8, 512, 100, 8, outs_arr(ok_y), E, need) == ERR["group"]
    assert lm(A, 8, 528, 16, 4, outs_arr(ok_y), E, need) == ERR["shape"]
    assert lm(A, 8, 512, 256, 5, outs_arr(ok_y), E, need) == ERR["dtype"]
    assert lm(NUL, 8, 512, 256, 8, outs_arr(ok_y), E, need) == ERR["null"]
    assert lm(A, 8, 512, 256, 8, outs_arr(ok_y), MIS, need) == ERR["align"]
    assert lm(NUL, 0, 512, 256, 8, outs_arr(ok_y), NUL, 0) == 0


def test_single_gemm_tile_count_bound(L):
    """M and N each within 2^30 but too many 128 x 128 tiles together."""
    assert gemm(A, B, C, 8, D, 1 << 30, 1 << 20, 64, E, NUL) == ERR["shape"]


def test_dequant_path_validation(L):
    Lb = cr.load()
    dq = lambda w, wb, s, N, K, g, o: Lb.convrot_dequantize_weight(w, wb, s, N, K, g, o, S0)
    gb = lambda x, w, M, N, K, y: Lb.convrot_gemm_bf16(x, w, M, N, K, y, S0)
    dl = lambda x, M, K, w, wb, s, N, g, y, ws, wsb: Lb.convrot_dequant_linear(x, M, K, w, wb, s, N, g, y, ws, wsb, S0)
    assert dq(A, 3, B, 4, 256, 256, C) == ERR["dtype"]
    assert dq(A, 8, B, 4, 250, 256, C) == ERR["shape"]
    assert dq(A, 4, B, 4, 272, 16, C) == ERR["shape"]       # int4 needs K % 32
    assert dq(A, 8, B, 4, 256, 3, C) == ERR["group"]
    assert dq(A, 8, B, -1, 256, 256, C) == ERR["shape"]
    assert dq(NUL, 8, B, 4, 256, 256, C) == ERR["null"]
    assert dq(A, 8, B, 4, 256, 256, MIS) == ERR["align"]
    assert dq(NUL, 8, NUL, 0, 256, 256, NUL) == 0
    assert gb(A, B, 4, 0, 64, C) == ERR["shape"]
    assert gb(A, B, 4, 4, 40, C) == ERR["shape"]
    assert gb(A, B, 4, 4, 65536, C) == ERR["shape"]
    assert gb(A, NUL, 4, 4, 64, C) == ERR["null"]
    assert gb(A, B, 4, 4, 64, MIS) == ERR["align"]
    assert gb(NUL, NUL, 0, 4, 64, NUL) == 0
    assert cr.convrot_dequant_workspace_size(0, 64) == 0
    assert cr.convrot_dequant_workspace_size(3, 64) == 512
    need = cr.convrot_dequant_workspace_size(64, 512)
    assert dl(A, 8, 512, B, 8, C, 64, 256, D, E, need - 1) == ERR["ws"]
    assert dl(A, 8, 512, B, 5, C, 64, 256, D, E, need) == ERR["dtype"]
    assert dl(A, 8, 512, B, 8, NUL, 64, 256, D, E, need) == ERR["null"]
    assert dl(A, 8, 512, B, 8, C, 64, 256, D, MIS, need) == ERR["align"]
    assert dl(NUL, 0, 512, NUL, 8, NUL, 64, 256, NUL, NUL, 0) == 0


def test_noalloc_validation(L):
    """The allocation-free linear checks its arguments like the others and
    refuses an input larger than its scratch area before any HIP call."""
    na = lambda x, M, K, w, s, N, g, y: cr.load().convrot_w8a8_linear_noalloc(x, M, K, w, s, N, g, y, S0)
    assert na(A, 8, 512, B, C, 0, 256, D) == ERR["shape"]
    assert na(A, 8, 500, B, C, 64, 256, D) == ERR["shape"]
    assert na(A, 8, 512, B, C, 64, 100, D) == ERR["group"]
    assert na(A, 8, 512, NUL, C, 64, 256, D) == ERR["null"]
    assert na(A, 8, 512, B, C, 64, 256, MIS) == ERR["align"]
    assert na(NUL, 0, 512, NUL, NUL, 64, 256, NUL) == 0
    K = 4096
    M = cr.NOALLOC_SCRATCH_BYTES // K                 # the codes fill the area, the scales do not fit
    assert cr.convrot_workspace_size(M, K) > cr.NOALLOC_SCRATCH_BYTES
    assert na(A, M, K, B, C, 64, 256, D) == ERR["scratch"]
