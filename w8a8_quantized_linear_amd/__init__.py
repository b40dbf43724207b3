"""ConvRot W8A8 / W4A8 quantized linear for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/convrot.h`` (``libconvrot.so``,
hand-written HIP kernels).  This module only marshals arguments: torch is used
for device memory and the current stream, every step of the computation runs
in the library's kernels.  There is no CPU fallback: if the library is not
built, or no GPU is visible, every call raises.

The functions named ``convrot_*`` mirror the C entry points one to one
(device pointers as tensors, same argument order); the short names below them
(``quantize_weight``, ``rotate_quant``, ``w8a8_linear``, ...) allocate the
outputs and return them.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "library_path", "ConvRotError", "LinearOut", "MAX_OUTS",
    "convrot_quantize_weight", "convrot_quantize_weight_i4_clip", "convrot_rotate_quant",
    "convrot_rmsnorm_rotate_quant", "convrot_workspace_size", "convrot_w8a8_linear", "convrot_w4a8_linear",
    "convrot_gemm_i8", "convrot_gemm_i8_multi", "convrot_linear_multi", "convrot_dequantize_weight",
    "convrot_gemm_bf16", "convrot_dequant_workspace_size", "convrot_dequant_linear",
    "convrot_w8a8_linear_noalloc", "convrot_status_string", "convrot_version", "NOALLOC_SCRATCH_BYTES",
    "quantize_weight", "rotate_quant", "rmsnorm_rotate_quant", "w8a8_linear", "w4a8_linear", "gemm_i8",
    "gemm_i8_multi", "linear_multi", "dequantize_weight", "gemm_bf16", "dequant_linear", "workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libconvrot.so")
_lib = None

OK = 0
W_F32, W_BF16 = 0, 1
MAX_K = 32768
MAX_OUTS = 8
NOALLOC_SCRATCH_BYTES = 64 << 20


class LinearOut(ctypes.Structure):
    """convrot_linear_out: one weight matrix of a multi-output call."""
    _fields_ = [("wq", ctypes.c_void_p), ("w_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("acc_out", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class ConvRotError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status}: {text}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libconvrot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m w8a8_quantized_linear_amd.build` "
            "(or __graft_entry__.build()) first")
    # torch first, where it is installed: it bundles its own HIP runtime
    # under the same soname as ROCm's, so whichever loads first serves the
    # process; loading this library first would put torch on ROCm's copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I, SZ, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    sigs = {
        "convrot_quantize_weight": (I, [P, I, I64, I64, I, I, P, P, P]),
        "convrot_quantize_weight_i4_clip": (I, [P, I, I64, I64, I, P, P, P, P]),
        "convrot_rotate_quant": (I, [P, I64, I64, I, P, P, P]),
        "convrot_rmsnorm_rotate_quant": (I, [P, P, F, I64, I64, I, P, P, P, P]),
        "convrot_workspace_size": (SZ, [I64, I64]),
        "convrot_w8a8_linear": (I, [P, I64, I64, P, P, I64, I, P, P, SZ, P]),
        "convrot_w4a8_linear": (I, [P, I64, I64, P, P, I64, I, P, P, SZ, P]),
        "convrot_gemm_i8": (I, [P, P, P, I, P, I64, I64, I64, P, P, P]),
        "convrot_gemm_i8_multi": (I, [P, P, I, I64, I64, P, I, P]),
        "convrot_linear_multi": (I, [P, I64, I64, I, I, P, I, P, SZ, P]),
        "convrot_dequantize_weight": (I, [P, I, P, I64, I64, I, P, P]),
        "convrot_gemm_bf16": (I, [P, P, I64, I64, I64, P, P]),
        "convrot_dequant_workspace_size": (SZ, [I64, I64]),
        "convrot_dequant_linear": (I, [P, I64, I64, P, I, P, I64, I, P, P, SZ, P]),
        "convrot_w8a8_linear_noalloc": (I, [P, I64, I64, P, P, I64, I, P, P]),
        "convrot_status_string": (ctypes.c_char_p, [I]),
        "convrot_version": (I, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    """Names the binding expects the library to export."""
    return ["convrot_quantize_weight", "convrot_quantize_weight_i4_clip", "convrot_rotate_quant",
            "convrot_rmsnorm_rotate_quant", "convrot_workspace_size", "convrot_w8a8_linear",
            "convrot_w4a8_linear", "convrot_gemm_i8", "convrot_gemm_i8_multi", "convrot_linear_multi",
            "convrot_dequantize_weight", "convrot_gemm_bf16", "convrot_dequant_workspace_size",
            "convrot_dequant_linear", "convrot_w8a8_linear_noalloc", "convrot_status_string", "convrot_version"]


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _dptr(t):
    """Device pointer of a tensor (None -> NULL); the tensor must be on a GPU."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("convrot: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("convrot: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _need(t, nbytes, what):
    """The library reads or writes nbytes of t: refuse a smaller buffer here,
    since the C layer cannot see buffer lengths."""
    if t is not None and _nbytes(t) < nbytes:
        raise ValueError(f"convrot: {what} holds {_nbytes(t)} bytes, the call touches {nbytes}")


def _expect(t, what, shape, dtypes):
    """Shape and dtype check of one argument of an allocating helper."""
    if t is None:
        raise ValueError(f"convrot: {what} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"convrot: {what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"convrot: {what} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"convrot: tensors on several devices: {sorted(str(d) for d in devs)}")


def _weight_shape(wbits, N, K):
    torch = _torch()
    if wbits == 8:
        return (N, K), (torch.int8,)
    if wbits == 4:
        if K % 2:
            raise ValueError("convrot: int4 weights need an even K")
        return (N, K // 2), (torch.uint8,)
    raise ValueError(f"convrot: wbits must be 8 or 4, got {wbits}")


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bits16(t):
    """bf16 tensor -> same storage viewed as int16 (raw bit patterns)."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"convrot: expected a bfloat16 tensor, got {t.dtype}")


def _check(fn: str, rc: int):
    if rc != OK:
        raise ConvRotError(fn, rc, convrot_status_string(rc))


# --------------------------------------------- C entry points, same names

def convrot_status_string(status: int) -> str:
    return load().convrot_status_string(int(status)).decode()


def convrot_version() -> int:
    return int(load().convrot_version())


def convrot_workspace_size(M: int, K: int) -> int:
    return int(load().convrot_workspace_size(int(M), int(K)))


def convrot_quantize_weight(w, w_dtype, N, K, group, bits, wq, w_scale, stream=None) -> int:
    if N > 0 and K > 0:
        _need(w, N * K * (4 if w_dtype == W_F32 else 2), "w")
        _need(wq, N * K // (2 if bits == 4 else 1), "wq")
        _need(w_scale, 4 * N, "w_scale")
    return load().convrot_quantize_weight(_dptr(w), int(w_dtype), int(N), int(K), int(group), int(bits),
                                          _dptr(wq), _dptr(w_scale), _stream(stream))


def convrot_quantize_weight_i4_clip(w, w_dtype, N, K, group, wq4, w_scale, clip_index, stream=None) -> int:
    if N > 0 and K > 0:
        _need(w, N * K * (4 if w_dtype == W_F32 else 2), "w")
        _need(wq4, N * K // 2, "wq4")
        _need(w_scale, 4 * N, "w_scale")
        _need(clip_index, 4 * N, "clip_index")
    return load().convrot_quantize_weight_i4_clip(_dptr(w), int(w_dtype), int(N), int(K), int(group),
                                                  _dptr(wq4), _dptr(w_scale), _dptr(clip_index),
                                                  _stream(stream))


def convrot_rotate_quant(x, M, K, group, xq, x_scale, stream=None) -> int:
    if M > 0 and K > 0:
        _need(x, 2 * M * K, "x")
        _need(xq, M * K, "xq")
        _need(x_scale, 4 * M, "x_scale")
    return load().convrot_rotate_quant(_dptr(x), int(M), int(K), int(group), _dptr(xq), _dptr(x_scale),
                                       _stream(stream))


def convrot_rmsnorm_rotate_quant(x, norm_w, eps, M, K, group, xq, x_scale, y_norm=None, stream=None) -> int:
    if M > 0 and K > 0:
        _need(x, 2 * M * K, "x")
        _need(norm_w, 4 * K, "norm_w")
        _need(xq, M * K, "xq")
        _need(x_scale, 4 * M, "x_scale")
        _need(y_norm, 2 * M * K, "y_norm")
    return load().convrot_rmsnorm_rotate_quant(_dptr(x), _dptr(norm_w), float(eps), int(M), int(K), int(group),
                                               _dptr(xq), _dptr(x_scale), _dptr(y_norm), _stream(stream))


def _need_linear(x, M, K, wq, w_bytes, w_scale, N, y, workspace, workspace_bytes):
    if M > 0 and K > 0 and N > 0:
        _need(x, 2 * M * K, "x")
        _need(wq, w_bytes, "wq")
        _need(w_scale, 4 * N, "w_scale")
        _need(y, 2 * M * N, "y")
        _need(workspace, workspace_bytes, "workspace")


def convrot_w8a8_linear(x, M, K, wq, w_scale, N, group, y, workspace, workspace_bytes, stream=None) -> int:
    _need_linear(x, M, K, wq, N * K, w_scale, N, y, workspace, workspace_bytes)
    return load().convrot_w8a8_linear(_dptr(x), int(M), int(K), _dptr(wq), _dptr(w_scale), int(N), int(group),
                                      _dptr(y), _dptr(workspace), int(workspace_bytes), _stream(stream))


def convrot_w8a8_linear_noalloc(x, M, K, wq, w_scale, N, group, y, stream=None) -> int:
    if M > 0 and K > 0 and N > 0:
        _need(x, 2 * M * K, "x")
        _need(wq, N * K, "wq")
        _need(w_scale, 4 * N, "w_scale")
        _need(y, 2 * M * N, "y")
    return load().convrot_w8a8_linear_noalloc(_dptr(x), int(M), int(K), _dptr(wq), _dptr(w_scale), int(N),
                                              int(group), _dptr(y), _stream(stream))


def convrot_w4a8_linear(x, M, K, wq4, w_scale, N, group, y, workspace, workspace_bytes, stream=None) -> int:
    _need_linear(x, M, K, wq4, N * K // 2, w_scale, N, y, workspace, workspace_bytes)
    return load().convrot_w4a8_linear(_dptr(x), int(M), int(K), _dptr(wq4), _dptr(w_scale), int(N), int(group),
                                      _dptr(y), _dptr(workspace), int(workspace_bytes), _stream(stream))


def convrot_gemm_i8(xq, x_scale, wq, wbits, w_scale, M, N, K, acc_out, y, stream=None) -> int:
    if M > 0 and N > 0 and K > 0:
        _need(xq, M * K, "xq")
        _need(x_scale, 4 * M, "x_scale")
        _need(wq, N * K // (2 if wbits == 4 else 1), "wq")
        _need(w_scale, 4 * N, "w_scale")
        _need(acc_out, 4 * M * N, "acc_out")
        _need(y, 2 * M * N, "y")
    return load().convrot_gemm_i8(_dptr(xq), _dptr(x_scale), _dptr(wq), int(wbits), _dptr(w_scale), int(M),
                                  int(N), int(K), _dptr(acc_out), _dptr(y), _stream(stream))


def convrot_dequantize_weight(wq, wbits, w_scale, N, K, group, w_out, stream=None) -> int:
    if N > 0 and K > 0:
        _need(wq, N * K // (2 if wbits == 4 else 1), "wq")
        _need(w_scale, 4 * N, "w_scale")
        _need(w_out, 2 * N * K, "w_out")
    return load().convrot_dequantize_weight(_dptr(wq), int(wbits), _dptr(w_scale), int(N), int(K), int(group),
                                            _dptr(w_out), _stream(stream))


def convrot_gemm_bf16(x, w, M, N, K, y, stream=None) -> int:
    if M > 0 and N > 0 and K > 0:
        _need(x, 2 * M * K, "x")
        _need(w, 2 * N * K, "w")
        _need(y, 2 * M * N, "y")
    return load().convrot_gemm_bf16(_dptr(x), _dptr(w), int(M), int(N), int(K), _dptr(y), _stream(stream))


def convrot_dequant_workspace_size(N: int, K: int) -> int:
    return int(load().convrot_dequant_workspace_size(int(N), int(K)))


def convrot_dequant_linear(x, M, K, wq, wbits, w_scale, N, group, y, workspace, workspace_bytes, stream=None) -> int:
    _need_linear(x, M, K, wq, N * K // (2 if wbits == 4 else 1), w_scale, N, y, workspace, workspace_bytes)
    return load().convrot_dequant_linear(_dptr(x), int(M), int(K), _dptr(wq), int(wbits), _dptr(w_scale), int(N),
                                         int(group), _dptr(y), _dptr(workspace), int(workspace_bytes),
                                         _stream(stream))


def _outs_array(outs, M=0, K=0, wbits=8):
    """Sequence of (wq, w_scale, N, acc_out, y) (tensors or None, and N) ->
    ctypes array of LinearOut (each buffer checked against M, K and N)."""
    if M > 0 and K > 0:
        for wq, ws, n, acc, y in outs:
            if n > 0:
                _need(wq, n * K // (2 if wbits == 4 else 1), "wq")
                _need(ws, 4 * n, "w_scale")
                _need(acc, 4 * M * n, "acc_out")
                _need(y, 2 * M * n, "y")
    arr = (LinearOut * max(1, len(outs)))()
    for i, (wq, ws, n, acc, y) in enumerate(outs):
        arr[i] = LinearOut(_dptr(wq), _dptr(ws), int(n), _dptr(acc), _dptr(y))
    return arr


def convrot_gemm_i8_multi(xq, x_scale, wbits, M, K, outs, stream=None) -> int:
    """outs: sequence of (wq, w_scale, N, acc_out, y)."""
    if M > 0 and K > 0:
        _need(xq, M * K, "xq")
        _need(x_scale, 4 * M, "x_scale")
    arr = _outs_array(outs, M, K, wbits)
    return load().convrot_gemm_i8_multi(_dptr(xq), _dptr(x_scale), int(wbits), int(M), int(K), arr, len(outs),
                                        _stream(stream))


def convrot_linear_multi(x, M, K, group, wbits, outs, workspace, workspace_bytes, stream=None) -> int:
    """outs: sequence of (wq, w_scale, N, acc_out, y)."""
    if M > 0 and K > 0:
        _need(x, 2 * M * K, "x")
        _need(workspace, workspace_bytes, "workspace")
    arr = _outs_array(outs, M, K, wbits)
    return load().convrot_linear_multi(_dptr(x), int(M), int(K), int(group), int(wbits), arr, len(outs),
                                       _dptr(workspace), int(workspace_bytes), _stream(stream))


# ----------------------------------------------------- allocating helpers
# Each checks its tensors' shapes, dtypes and device before anything reaches
# the library (ValueError on a mismatch), then allocates what it returns.

def _mk(x, dtypes=None, what="x"):
    """[M, K] of a 2-D activation-like tensor (bf16 bits by default)."""
    if x.dim() != 2:
        raise ValueError(f"convrot: {what} must be 2-D [M, K], got shape {tuple(x.shape)}")
    dtypes = dtypes or _bf16_types()
    if x.dtype not in dtypes:
        raise ValueError(f"convrot: {what} has dtype {x.dtype}, expected one of {[str(d) for d in dtypes]}")
    return int(x.shape[0]), int(x.shape[1])


def _check_weight(wq, w_scale, wbits, K, what):
    """wq is int8 [N, K] (wbits 8) or packed uint8 [N, K/2] (wbits 4), with
    an fp32 [N] scale."""
    torch = _torch()
    if wq.dim() != 2:
        raise ValueError(f"convrot: {what} must be 2-D, got shape {tuple(wq.shape)}")
    N = int(wq.shape[0])
    shape, dtypes = _weight_shape(wbits, N, K)
    _expect(wq, what, shape, dtypes)
    _expect(w_scale, f"{what} scale", (N,), (torch.float32,))


def _check_ws(ws, nbytes):
    torch = _torch()
    if ws.dtype not in (torch.uint8, torch.int8) or ws.dim() != 1:
        raise ValueError("convrot: the workspace must be a 1-D uint8 tensor")
    if ws.numel() < nbytes:
        raise ValueError(f"convrot: workspace of {ws.numel()} bytes, the call needs {nbytes}")



def quantize_weight(w, group: int = 256, bits: int = 8, with_clip_index: bool = False):
    """w fp32/bf16 [N, K] on the GPU -> (wq, w_scale[, clip_index]).
    bits 8: wq int8 [N, K]; bits 4: wq uint8 [N, K/2] (two nibbles per byte)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError(f"convrot.quantize_weight: w must be 2-D [N, K], got shape {tuple(w.shape)}")
    N, K = w.shape
    if w.dtype == torch.float32:
        wd = W_F32
    elif w.dtype == torch.bfloat16:
        wd = W_BF16
    else:
        raise TypeError("convrot.quantize_weight: w must be float32 or bfloat16")
    _weight_shape(bits, N, K)
    dev = w.device
    scale = torch.empty((N,), dtype=torch.float32, device=dev)
    if bits == 8:
        wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    else:
        wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if bits == 4 and with_clip_index:
        ci = torch.empty((N,), dtype=torch.int32, device=dev)
        _check("convrot_quantize_weight_i4_clip",
               convrot_quantize_weight_i4_clip(w, wd, N, K, group, wq, scale, ci))
        return wq, scale, ci
    _check("convrot_quantize_weight", convrot_quantize_weight(w, wd, N, K, group, bits, wq, scale))
    return wq, scale


def rotate_quant(x, group: int = 256):
    """x bf16 [M, K] -> (xq int8 [M, K], x_scale fp32 [M])."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("convrot_rotate_quant", convrot_rotate_quant(x, M, K, group, xq, xs))
    return xq, xs


def rmsnorm_rotate_quant(x, norm_w, eps: float = 1e-6, group: int = 256, want_y: bool = False):
    """RMSNorm with (1 + norm_w) weights fused with rotate_quant.
    x bf16 [M, K], norm_w fp32 [K] -> (xq int8 [M, K], x_scale fp32 [M][, y bf16 [M, K]])."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    _expect(norm_w, "norm_w", (K,), (torch.float32,))
    _same_device(x, norm_w)
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if want_y else None
    _check("convrot_rmsnorm_rotate_quant",
           convrot_rmsnorm_rotate_quant(x, norm_w, eps, M, K, group, xq, xs, y))
    return (xq, xs, y) if want_y else (xq, xs)


def linear_multi(x, weights, wbits: int = 8, group: int = 256, outs=None, ws=None):
    """Several linears on one input (rotated and quantized once, one GEMM
    launch).  weights: sequence of (wq, w_scale); returns the list of bf16
    outputs [M, N_o] (or fills ``outs``)."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    if not 1 <= len(weights) <= MAX_OUTS:
        raise ValueError(f"convrot.linear_multi: 1..{MAX_OUTS} weights, got {len(weights)}")
    for i, (wq, wsc) in enumerate(weights):
        _check_weight(wq, wsc, wbits, K, f"weights[{i}]")
    if outs is None:
        outs = [torch.empty((M, wq.shape[0]), dtype=torch.bfloat16, device=x.device) for wq, _ in weights]
    if len(outs) != len(weights):
        raise ValueError("convrot.linear_multi: one output per weight")
    for i, ((wq, _), y) in enumerate(zip(weights, outs)):
        _expect(y, f"outs[{i}]", (M, wq.shape[0]), _bf16_types())
    if ws is None:
        ws = workspace(M, K, x.device)
    _check_ws(ws, convrot_workspace_size(M, K))
    _same_device(x, ws, *[t for wq, wsc in weights for t in (wq, wsc)], *outs)
    desc = [(wq, wsc, wq.shape[0], None, y) for (wq, wsc), y in zip(weights, outs)]
    _check("convrot_linear_multi", convrot_linear_multi(x, M, K, group, wbits, desc, ws, ws.numel()))
    return outs


def gemm_i8_multi(xq, x_scale, weights, wbits: int = 8, want_acc: bool = True, want_y: bool = True):
    """convrot_gemm_i8 over several weight matrices sharing xq; returns a list
    of (acc int32 [M, N_o] or None, y bf16 [M, N_o] or None)."""
    torch = _torch()
    M, K = _mk(xq, (torch.int8,), "xq")
    _expect(x_scale, "x_scale", (M,), (torch.float32,))
    if not 1 <= len(weights) <= MAX_OUTS:
        raise ValueError(f"convrot.gemm_i8_multi: 1..{MAX_OUTS} weights, got {len(weights)}")
    for i, (wq, wsc) in enumerate(weights):
        _check_weight(wq, wsc, wbits, K, f"weights[{i}]")
    _same_device(xq, x_scale, *[t for wq, wsc in weights for t in (wq, wsc)])
    res, desc = [], []
    for wq, wsc in weights:
        n = wq.shape[0]
        acc = torch.empty((M, n), dtype=torch.int32, device=xq.device) if want_acc else None
        y = torch.empty((M, n), dtype=torch.bfloat16, device=xq.device) if want_y else None
        res.append((acc, y))
        desc.append((wq, wsc, n, acc, y))
    _check("convrot_gemm_i8_multi", convrot_gemm_i8_multi(xq, x_scale, wbits, M, K, desc))
    return res


def dequantize_weight(wq, w_scale, K: int, wbits: int = 8, group: int = 256):
    """Codes (int8 [N, K] or packed int4 uint8 [N, K/2]) -> bf16 weight [N, K]."""
    torch = _torch()
    N = wq.shape[0]
    _check_weight(wq, w_scale, wbits, K, "wq")
    _same_device(wq, w_scale)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=wq.device)
    _check("convrot_dequantize_weight", convrot_dequantize_weight(wq, wbits, w_scale, N, K, group, out))
    return out


def gemm_bf16(x, w, out=None):
    """bf16 x [M, K] . w [N, K]^T -> bf16 [M, N] (fp32 accumulation)."""
    torch = _torch()
    x, w = _bits16(x), _bits16(w)
    M, K = _mk(x)
    N = w.shape[0]
    _expect(w, "w", (N, K), _bf16_types())
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _expect(y, "out", (M, N), _bf16_types())
    _same_device(x, w, y)
    _check("convrot_gemm_bf16", convrot_gemm_bf16(x, w, M, N, K, y))
    return y


def dequant_linear(x, wq, w_scale, wbits: int = 8, group: int = 256, out=None, ws=None):
    """The weight-only linear: dequantize wq (into a workspace), then the bf16 matmul."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    N = wq.shape[0]
    _check_weight(wq, w_scale, wbits, K, "wq")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _expect(y, "out", (M, N), _bf16_types())
    if ws is None:
        ws = torch.empty((max(convrot_dequant_workspace_size(N, K), 16),), dtype=torch.uint8, device=x.device)
    _check_ws(ws, convrot_dequant_workspace_size(N, K))
    _same_device(x, wq, w_scale, y, ws)
    _check("convrot_dequant_linear",
           convrot_dequant_linear(x, M, K, wq, wbits, w_scale, N, group, y, ws, ws.numel()))
    return y


def workspace(M: int, K: int, device="cuda"):
    torch = _torch()
    n = convrot_workspace_size(M, K)
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device)


def w8a8_linear(x, wq, w_scale, group: int = 256, out=None, ws=None):
    """y = ConvRot W8A8 linear(x); x bf16 [M, K], wq int8 [N, K] -> y bf16 [M, N]."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    N = wq.shape[0]
    _check_weight(wq, w_scale, 8, K, "wq")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _expect(y, "out", (M, N), _bf16_types())
    if ws is None:
        ws = workspace(M, K, x.device)
    _check_ws(ws, convrot_workspace_size(M, K))
    _same_device(x, wq, w_scale, y, ws)
    _check("convrot_w8a8_linear",
           convrot_w8a8_linear(x, M, K, wq, w_scale, N, group, y, ws, ws.numel()))
    return y


def w4a8_linear(x, wq4, w_scale, group: int = 256, out=None, ws=None):
    """W4A8 variant; wq4 uint8 [N, K/2] -> y bf16 [M, N]."""
    torch = _torch()
    x = _bits16(x)
    M, K = _mk(x)
    N = wq4.shape[0]
    _check_weight(wq4, w_scale, 4, K, "wq4")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _expect(y, "out", (M, N), _bf16_types())
    if ws is None:
        ws = workspace(M, K, x.device)
    _check_ws(ws, convrot_workspace_size(M, K))
    _same_device(x, wq4, w_scale, y, ws)
    _check("convrot_w4a8_linear",
           convrot_w4a8_linear(x, M, K, wq4, w_scale, N, group, y, ws, ws.numel()))
    return y


def gemm_i8(xq, x_scale, wq, w_scale, wbits: int = 8, want_acc: bool = True, want_y: bool = True):
    """Integer product on given codes -> (acc int32 [M, N] or None, y bf16 [M, N] or None)."""
    torch = _torch()
    M, K = _mk(xq, (torch.int8,), "xq")
    N = wq.shape[0]
    if want_y or x_scale is not None:
        _expect(x_scale, "x_scale", (M,), (torch.float32,))
    if want_y or w_scale is not None:
        _check_weight(wq, w_scale, wbits, K, "wq")
    else:
        shape, dtypes = _weight_shape(wbits, N, K)
        _expect(wq, "wq", shape, dtypes)
    _same_device(xq, x_scale, wq, w_scale)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if want_acc else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if want_y else None
    _check("convrot_gemm_i8", convrot_gemm_i8(xq, x_scale, wq, wbits, w_scale, M, N, K, acc, y))
    return acc, y
