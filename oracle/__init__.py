"""CPU oracle for the ConvRot W8A8 / W4A8 linear -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow reference the HIP library is checked against.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it.  The library (``w8a8_quantized_linear_amd``) never imports, links
or calls anything here, and the two share no code.

The arithmetic lives in ``convrot_oracle.c`` (plain C, fp64 dense Hadamard
product, naive integer GEMM), compiled with gcc into ``liboracle.so``; this
module only marshals numpy arrays into it.  Every function cites the page
passage it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C11 + OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def use_library(path=None):
    """Point the binding at another build of the oracle source (the mutation
    tests use this to load deliberately broken copies); None restores the
    default library."""
    global _lib, _LIB_PATH
    _lib = None
    _LIB_PATH = path or os.path.join(_HERE, "liboracle.so")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    sigs = {
        "oracle_hadamard": (None, [I, P]),
        "oracle_rotate_rows": (I, [P, I64, I64, I, P]),
        "oracle_quantize_weight_i8": (I, [P, I64, I64, I, P, P]),
        "oracle_rotate_quant": (I, [P, I64, I64, I, P, P]),
        "oracle_gemm_i8": (I, [P, P, I64, I64, I64, P]),
        "oracle_epilogue": (I, [P, P, P, I64, I64, P]),
        "oracle_w8a8_linear": (I, [P, I64, I64, P, P, I64, I, P]),
        "oracle_quantize_weight_i4": (I, [P, I64, I64, I, P, P, P]),
        "oracle_quantize_weight_i4_ex": (I, [P, I64, I64, I, P, P, P, P, P]),
        "oracle_unpack_i4": (I, [P, I64, I64, P]),
        "oracle_w4a8_linear": (I, [P, I64, I64, P, P, I64, I, P]),
        "oracle_rmsnorm_bf16": (I, [P, P, ctypes.c_float, I64, I64, P]),
        "oracle_rmsnorm_rotate_quant": (I, [P, P, ctypes.c_float, I64, I64, I, P, P, P]),
        "oracle_dequantize_weight": (I, [P, P, I64, I64, I, P]),
        "oracle_gemm_bf16": (I, [P, P, I64, I64, I64, P]),
        "oracle_num_threads": (I, []),
        "oracle_set_num_threads": (None, [I]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == 2:
        raise OracleError(f"{what}: int32 accumulator overflow")
    if rc != 0:
        raise OracleError(f"{what}: invalid arguments (rc={rc})")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's row loops use from now on."""
    _load().oracle_set_num_threads(int(n))


def hadamard(g: int) -> np.ndarray:
    """Dense normalised Sylvester Hadamard matrix of order g (fp64)."""
    H = np.empty((g, g), dtype=np.float64)
    _load().oracle_hadamard(int(g), _ptr(H))
    return H


def rotate_rows(x: np.ndarray, group: int = 256) -> np.ndarray:
    """x fp64 [rows, K] -> x * blockdiag(H, ..., H) in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, K = x.shape
    out = np.empty_like(x)
    _check(_load().oracle_rotate_rows(_ptr(x), rows, K, int(group), _ptr(out)), "rotate_rows")
    return out


def quantize_weight_i8(w: np.ndarray, group: int = 256):
    """W fp32 [N, K] -> (wq int8 [N, K], w_scale fp32 [N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq = np.empty((N, K), dtype=np.int8)
    s = np.empty((N,), dtype=np.float32)
    _check(_load().oracle_quantize_weight_i8(_ptr(w), N, K, int(group), _ptr(wq), _ptr(s)),
           "quantize_weight_i8")
    return wq, s


def rotate_quant(x_bf16: np.ndarray, group: int = 256):
    """x bf16 bits (uint16) [M, K] -> (xq int8 [M, K], x_scale fp32 [M])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    _check(_load().oracle_rotate_quant(_ptr(x), M, K, int(group), _ptr(xq), _ptr(s)), "rotate_quant")
    return xq, s


def gemm_i8(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """int8 [M, K] x int8 [N, K] -> int32 [M, N] (sum over K)."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    assert K == K2
    acc = np.empty((M, N), dtype=np.int32)
    _check(_load().oracle_gemm_i8(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc)), "gemm_i8")
    return acc


def epilogue(acc: np.ndarray, x_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """int32 [M, N] -> bf16 bits uint16 [M, N]."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    xs = np.ascontiguousarray(x_scale, dtype=np.float32)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_epilogue(_ptr(acc), _ptr(xs), _ptr(ws), M, N, _ptr(y)), "epilogue")
    return y


def w8a8_linear(x_bf16: np.ndarray, wq: np.ndarray, w_scale: np.ndarray, group: int = 256) -> np.ndarray:
    """bf16 bits [M, K] -> bf16 bits [M, N]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x.shape
    N = wq.shape[0]
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_w8a8_linear(_ptr(x), M, K, _ptr(wq), _ptr(ws), N, int(group), _ptr(y)),
           "w8a8_linear")
    return y


def quantize_weight_i4(w: np.ndarray, group: int = 256, force_index=None, with_errors: bool = False):
    """W fp32 [N, K] -> (wq4 uint8 [N, K/2], w_scale fp32 [N], clip index int32 [N]
    [, errors fp64 [N, 51]]).

    force_index (int [N], values 0..50) makes row n take that clip candidate
    instead of the argmin; with_errors also returns every candidate's error."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq4 = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N,), dtype=np.float32)
    ci = np.empty((N,), dtype=np.int32)
    fi = None if force_index is None else np.ascontiguousarray(force_index, dtype=np.int32)
    if fi is not None:
        assert fi.shape == (N,)
    err = np.empty((N, 51), dtype=np.float64) if with_errors else None
    _check(_load().oracle_quantize_weight_i4_ex(_ptr(w), N, K, int(group), None if fi is None else _ptr(fi),
                                                _ptr(wq4), _ptr(s), _ptr(ci), None if err is None else _ptr(err)),
           "quantize_weight_i4")
    return (wq4, s, ci, err) if with_errors else (wq4, s, ci)


def unpack_i4(wq4: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> int8 codes [N, K] (signed nibbles, low nibble first)."""
    wq4 = np.ascontiguousarray(wq4, dtype=np.uint8)
    N, Kh = wq4.shape
    wq = np.empty((N, 2 * Kh), dtype=np.int8)
    _check(_load().oracle_unpack_i4(_ptr(wq4), N, 2 * Kh, _ptr(wq)), "unpack_i4")
    return wq


def w4a8_linear(x_bf16: np.ndarray, wq4: np.ndarray, w_scale: np.ndarray, group: int = 256) -> np.ndarray:
    """bf16 bits [M, K], packed int4 [N, K/2] -> bf16 bits [M, N]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    wq4 = np.ascontiguousarray(wq4, dtype=np.uint8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x.shape
    N = wq4.shape[0]
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_w4a8_linear(_ptr(x), M, K, _ptr(wq4), _ptr(ws), N, int(group), _ptr(y)),
           "w4a8_linear")
    return y


def rmsnorm(x_bf16: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm with (1 + w) weights: bf16 bits [M, K], fp32 [K] -> bf16 bits [M, K]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = x.shape
    assert w.shape == (K,)
    y = np.empty((M, K), dtype=np.uint16)
    _check(_load().oracle_rmsnorm_bf16(_ptr(x), _ptr(w), float(eps), M, K, _ptr(y)), "rmsnorm")
    return y


def rmsnorm_rotate_quant(x_bf16: np.ndarray, w: np.ndarray, eps: float = 1e-6, group: int = 256):
    """RMSNorm, then rotate + quantize its bf16 output -> (xq int8, x_scale fp32, y bf16 bits)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = x.shape
    assert w.shape == (K,)
    xq = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    y = np.empty((M, K), dtype=np.uint16)
    _check(_load().oracle_rmsnorm_rotate_quant(_ptr(x), _ptr(w), float(eps), M, K, int(group), _ptr(xq), _ptr(s),
                                               _ptr(y)), "rmsnorm_rotate_quant")
    return xq, s, y


def dequantize_weight(wq: np.ndarray, w_scale: np.ndarray, group: int = 256) -> np.ndarray:
    """Weight-only path: int8 codes [N, K] (or packed int4 uint8 [N, K/2]) and
    fp32 row scales -> the dequantized, un-rotated weight as bf16 bits [N, K]."""
    wq = np.ascontiguousarray(wq)
    if wq.dtype == np.uint8:
        wq = unpack_i4(wq)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    s = np.ascontiguousarray(w_scale, dtype=np.float32)
    N, K = wq.shape
    assert s.shape == (N,)
    out = np.empty((N, K), dtype=np.uint16)
    _check(_load().oracle_dequantize_weight(_ptr(wq), _ptr(s), N, K, int(group), _ptr(out)), "dequantize_weight")
    return out


def gemm_bf16(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """bf16 bits [M, K] x bf16 bits [N, K] -> bf16 bits [M, N] (fp64 sum, then fp32, then bf16)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_gemm_bf16(_ptr(x), _ptr(w), M, N, K, _ptr(y)), "gemm_bf16")
    return y


def dequant_linear(x_bf16: np.ndarray, wq: np.ndarray, w_scale: np.ndarray, group: int = 256) -> np.ndarray:
    """The weight-only linear: dequantize, then the bf16 matmul with the unrotated input."""
    return gemm_bf16(x_bf16, dequantize_weight(wq, w_scale, group))
