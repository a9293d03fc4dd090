"""bit_ptq_reconstruction_amd -- MI355X-native W4A4 Hadamard-rotated quantized linear layers.

This module is a thin ctypes binding of ``libqv.so`` (C ABI in ``include/qv.h``): it turns torch
tensors into device pointers, sizes, leading dimensions and the current HIP stream, and raises
``QVError`` on a non-OK status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback path.  Functions carry the C names.

Method (page "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), sections 训练后量化（PTQ） and
双平滑细粒度量化（DSFQ）): rotate activations and weights by a Hadamard matrix, smooth per channel in
the rotated space, quantize symmetrically to 4 bits (per token / per output channel), multiply in
integers and dequantize.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QVError", "QV_F32", "QV_BF16", "QV_EPI_NONE", "QV_EPI_GELU", "lib", "library_path",
    "qv_status_string", "qv_hadamard_smooth_quant", "qv_pack_weights", "qv_w4a4_gemm",
    "qv_w4a4_linear_workspace_size", "qv_w4a4_linear", "qv_w4a4_linear_noalloc", "qv_smooth_calibrate",
    "QV_NOALLOC_SCRATCH_BYTES", "qv_w4a4_gemm_requant", "qv_w4a4_gemm_requant_workspace_size",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libqv.so")

QV_F32, QV_BF16 = 0, 1
# Size of the library's static scratch array behind qv_w4a4_linear_noalloc (QV_NOALLOC_SCRATCH_BYTES
# in include/qv.h).
QV_NOALLOC_SCRATCH_BYTES = 32 << 20
QV_EPI_NONE, QV_EPI_GELU = 0, 1

_lib = None


class QVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {qv_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libqv.so (built in-tree by ``__graft_entry__.build()``); fail loudly if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def bind(L):
    """Declare the C signatures of every entry point on a loaded library handle and return it."""
    P, i64, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.qv_status_string.argtypes = [i32]
    L.qv_status_string.restype = ctypes.c_char_p
    L.qv_hadamard_smooth_quant.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
    L.qv_pack_weights.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
    L.qv_w4a4_gemm.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P, i32, i64, P]
    L.qv_w4a4_linear_workspace_size.argtypes = [i64, i64]
    L.qv_w4a4_linear_workspace_size.restype = sz
    L.qv_w4a4_linear.argtypes = [P, i32, i64, i64, i64, P, P, P, P, i64, i32, P, i32, i64, P, sz, P]
    L.qv_w4a4_linear_noalloc.argtypes = [P, i32, i64, i64, i64, P, P, P, P, i64, i32, P, i32, i64, P]
    L.qv_w4a4_gemm_requant_workspace_size.argtypes = [i64]
    L.qv_w4a4_gemm_requant_workspace_size.restype = sz
    L.qv_w4a4_gemm_requant.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P, i64, P, P, P, P, sz, P]
    L.qv_smooth_calibrate.argtypes = [P, i32, i64, i64, P, i32, i64, i64, i64, f32, P, P, P]
    L.qv_hadamard_smooth_quant8.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
    L.qv_pack_weights8.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
    L.qv_w8a8_gemm.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P, i32, i64, P]
    L.qv_w8a8_linear_workspace_size.argtypes = [i64, i64]
    L.qv_w8a8_linear_workspace_size.restype = sz
    L.qv_w8a8_linear.argtypes = [P, i32, i64, i64, i64, P, P, P, P, i64, i32, P, i32, i64, P, sz, P]
    L.qv_hadamard_smooth_quant_grouped.argtypes = [P, i32, i64, i64, i64, P, i64, P, P, P]
    L.qv_pack_weights_grouped.argtypes = [P, i32, i64, i64, i64, P, i64, P, P, P]
    L.qv_w4a4_gemm_grouped.argtypes = [P, P, P, P, P, i64, i64, i64, i64, i32, P, i32, i64, P]
    L.qv_w4a4_linear_grouped_workspace_size.argtypes = [i64, i64, i64]
    L.qv_w4a4_linear_grouped_workspace_size.restype = sz
    L.qv_w4a4_linear_grouped.argtypes = [P, i32, i64, i64, i64, P, i64, P, P, P, i64, i32, P, i32, i64, P, sz,
                                         P]
    for name in ("qv_hadamard_smooth_quant", "qv_pack_weights", "qv_w4a4_gemm", "qv_w4a4_linear",
                 "qv_w4a4_linear_noalloc", "qv_w4a4_gemm_requant", "qv_smooth_calibrate", "qv_hadamard_smooth_quant8", "qv_pack_weights8", "qv_w8a8_gemm",
                 "qv_w8a8_linear", "qv_hadamard_smooth_quant_grouped", "qv_pack_weights_grouped",
                 "qv_w4a4_gemm_grouped", "qv_w4a4_linear_grouped"):
        getattr(L, name).restype = i32
    return L


def qv_status_string(status: int) -> str:
    return lib().qv_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QVError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return QV_F32
    if t.dtype == torch.bfloat16:
        return QV_BF16
    raise ValueError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


# ----------------------------------------------------------------------------- argument checks
# The C ABI receives bare pointers and cannot see how large a buffer is, so the binding checks every
# tensor against the sizes the call implies before anything reaches the library: an undersized or
# strided operand would otherwise be read or written past its end by the kernels.  Every failed
# check raises ValueError and nothing is launched.

_FLOAT = ("float32", "bfloat16")


def _dtname(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _spec(what: str, name: str, t, dtypes, shape, rows_packed: bool = False, optional: bool = False):
    """Check one operand: its dtype is one of ``dtypes``; its shape equals ``shape``; it is dense
    (``rows_packed``: only the column stride must be 1, rows may be padded).  Returns the tensor."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{what}: {name} is required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "dtype"):
        raise ValueError(f"{what}: {name} must be a torch tensor")
    if _dtname(t) not in dtypes:
        raise ValueError(f"{what}: {name} has dtype {_dtname(t)}, expected {' or '.join(dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if rows_packed:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or t.stride(0) < t.shape[1]:
            raise ValueError(f"{what}: {name} needs unit column stride and a row stride of at least its width")
    elif not t.is_contiguous():
        raise ValueError(f"{what}: {name} must be contiguous")
    return t


def _same_gpu(what: str, *tensors) -> None:
    """All operands on one GPU (checked after the shapes, so shape errors are reported first)."""
    ts = [t for t in tensors if t is not None]
    for t in ts:
        if not t.is_cuda:
            raise ValueError(f"{what}: every operand must be a GPU tensor (got one on {t.device})")
    if len({t.device for t in ts}) > 1:
        raise ValueError(f"{what}: operands are on different devices {sorted({str(t.device) for t in ts})}")


def _rows_cols(what: str, name: str, t):
    if not hasattr(t, "shape") or len(t.shape) != 2:
        raise ValueError(f"{what}: {name} must be a 2-D tensor")
    return int(t.shape[0]), int(t.shape[1])


def _check_rotate_quant(what, X, mult, q, scale, code_cols, scale_shape):
    M, K = _rows_cols(what, "X", X)
    _spec(what, "X", X, _FLOAT, (M, K), rows_packed=True)
    _spec(what, "multiplier", mult, ("float32",), (K,), optional=True)
    _spec(what, "codes", q, ("uint8",) if code_cols(K) != K else ("int8",), (M, code_cols(K)))
    _spec(what, "scales", scale, ("float32",), scale_shape(M, K))
    _same_gpu(what, X, mult, q, scale)
    return M, K


def _check_gemm(what, Xq, xs, Wq, ws, bias, Y, code_dtype, k_of, scale_cols=None):
    M, kc = _rows_cols(what, "Xq", Xq)
    N = _rows_cols(what, "Wq", Wq)[0]
    K = k_of(kc)
    _spec(what, "Xq", Xq, (code_dtype,), (M, kc))
    _spec(what, "Wq", Wq, (code_dtype,), (N, kc))
    _spec(what, "x_scale", xs, ("float32",), (M,) if scale_cols is None else (M, scale_cols(K)))
    _spec(what, "w_scale", ws, ("float32",), (N,) if scale_cols is None else (N, scale_cols(K)))
    _spec(what, "bias", bias, ("float32",), (N,), optional=True)
    _spec(what, "Y", Y, _FLOAT, (M, N), rows_packed=True)
    _same_gpu(what, Xq, xs, Wq, ws, bias, Y)
    return M, N, K


def _check_workspace(what, workspace, need: int):
    _spec(what, "workspace", workspace, ("uint8",), (workspace.numel(),) if workspace is not None else (0,))
    if workspace.numel() < need:
        raise ValueError(f"{what}: workspace holds {workspace.numel()} bytes, needs {need}")


def qv_hadamard_smooth_quant(X, inv_smooth, Xq, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq [M, K/2] uint8 (packed int4), x_scale [M] fp32."""
    M, K = _check_rotate_quant("qv_hadamard_smooth_quant", X, inv_smooth, Xq, x_scale, lambda K: K // 2,
                               lambda M, K: (M,))
    _check(lib().qv_hadamard_smooth_quant(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Xq),
                                          _ptr(x_scale), _stream(stream)), "qv_hadamard_smooth_quant")


def qv_pack_weights(W, smooth, Wq, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq [N, K/2] uint8 (packed int4), w_scale [N] fp32."""
    N, K = _check_rotate_quant("qv_pack_weights", W, smooth, Wq, w_scale, lambda K: K // 2, lambda M, K: (M,))
    _check(lib().qv_pack_weights(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), _ptr(Wq), _ptr(w_scale),
                                 _stream(stream)), "qv_pack_weights")


def qv_w4a4_gemm(Xq, x_scale, Wq, w_scale, bias, Y, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] (fp32/bf16) = dequant(Xq . Wq^T) (+ bias) (+ GELU)."""
    M, N, K = _check_gemm("qv_w4a4_gemm", Xq, x_scale, Wq, w_scale, bias, Y, "uint8", lambda c: 2 * c)
    _check(lib().qv_w4a4_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, K, int(epi),
                              _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)), "qv_w4a4_gemm")


def qv_w4a4_linear_workspace_size(M: int, K: int) -> int:
    return int(lib().qv_w4a4_linear_workspace_size(int(M), int(K)))


def qv_w4a4_linear(X, inv_smooth, Wq, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE, stream=None) -> None:
    """The whole online layer; ``workspace`` is a uint8 device tensor of at least
    ``qv_w4a4_linear_workspace_size(M, K)`` bytes."""
    what = "qv_w4a4_linear"
    M, K = _rows_cols(what, "X", X)
    N = _rows_cols(what, "Wq", Wq)[0]
    _spec(what, "X", X, _FLOAT, (M, K), rows_packed=True)
    _spec(what, "inv_smooth", inv_smooth, ("float32",), (K,), optional=True)
    _spec(what, "Wq", Wq, ("uint8",), (N, K // 2))
    _spec(what, "w_scale", w_scale, ("float32",), (N,))
    _spec(what, "bias", bias, ("float32",), (N,), optional=True)
    _spec(what, "Y", Y, _FLOAT, (M, N), rows_packed=True)
    _check_workspace(what, workspace, qv_w4a4_linear_workspace_size(M, K))
    _same_gpu(what, X, inv_smooth, Wq, w_scale, bias, Y, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w4a4_linear(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Wq), _ptr(w_scale),
                                _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y), _ptr(workspace), nbytes,
                                _stream(stream)), "qv_w4a4_linear")


def qv_w4a4_gemm_requant_workspace_size(M: int) -> int:
    return int(lib().qv_w4a4_gemm_requant_workspace_size(int(M)))


def qv_w4a4_gemm_requant(Xq, x_scale, Wq, w_scale, bias, Y, inv_smooth_next, Xq_next, x_scale_next, workspace,
                         epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] bf16 = dequant(Xq . Wq^T) (+ bias) (+ GELU), and Xq_next [M, N/2] / x_scale_next [M]: Y's
    rows rotated at width N (1024 or 4096), smoothed by ``inv_smooth_next`` and quantized to int4, as
    ``qv_hadamard_smooth_quant(Y, inv_smooth_next, ...)`` would give."""
    what = "qv_w4a4_gemm_requant"
    M, N, K = _check_gemm(what, Xq, x_scale, Wq, w_scale, bias, Y, "uint8", lambda c: 2 * c)
    if _dtname(Y) != "bfloat16":
        raise ValueError(f"{what}: Y must be bfloat16 (the next layer's input)")
    _spec(what, "inv_smooth_next", inv_smooth_next, ("float32",), (N,), optional=True)
    _spec(what, "Xq_next", Xq_next, ("uint8",), (M, N // 2))
    _spec(what, "x_scale_next", x_scale_next, ("float32",), (M,))
    _check_workspace(what, workspace, qv_w4a4_gemm_requant_workspace_size(M))
    _same_gpu(what, Xq, x_scale, Wq, w_scale, bias, Y, inv_smooth_next, Xq_next, x_scale_next, workspace)
    _check(lib().qv_w4a4_gemm_requant(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, K, int(epi),
                                      _ptr(Y), _ld(Y), _ptr(inv_smooth_next), _ptr(Xq_next), _ptr(x_scale_next),
                                      _ptr(workspace), workspace.numel(), _stream(stream)), what)


def qv_w4a4_linear_noalloc(X, inv_smooth, Wq, w_scale, bias, Y, epi: int = QV_EPI_NONE, stream=None) -> None:
    """The whole online layer without a caller workspace: the codes and scales live in the library's
    static device array (at most ``QV_NOALLOC_SCRATCH_BYTES`` of them).  Calls that overlap in time
    on one GPU race on that array; calls on one stream are ordered."""
    what = "qv_w4a4_linear_noalloc"
    M, K = _rows_cols(what, "X", X)
    N = _rows_cols(what, "Wq", Wq)[0]
    _spec(what, "X", X, _FLOAT, (M, K), rows_packed=True)
    _spec(what, "inv_smooth", inv_smooth, ("float32",), (K,), optional=True)
    _spec(what, "Wq", Wq, ("uint8",), (N, K // 2))
    _spec(what, "w_scale", w_scale, ("float32",), (N,))
    _spec(what, "bias", bias, ("float32",), (N,), optional=True)
    _spec(what, "Y", Y, _FLOAT, (M, N), rows_packed=True)
    _same_gpu(what, X, inv_smooth, Wq, w_scale, bias, Y)
    _check(lib().qv_w4a4_linear_noalloc(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Wq),
                                        _ptr(w_scale), _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y),
                                        _stream(stream)), what)


def qv_smooth_calibrate(Xc, W, smooth, inv_smooth, alpha: float = 0.5, stream=None) -> None:
    """smooth [K], inv_smooth [K] fp32 from the rotated calibration rows Xc [Mc, K] and weights W [N, K]."""
    what = "qv_smooth_calibrate"
    Mc, K = _rows_cols(what, "Xc", Xc)
    N = _rows_cols(what, "W", W)[0]
    _spec(what, "Xc", Xc, _FLOAT, (Mc, K), rows_packed=True)
    _spec(what, "W", W, _FLOAT, (N, K), rows_packed=True)
    _spec(what, "smooth", smooth, ("float32",), (K,))
    _spec(what, "inv_smooth", inv_smooth, ("float32",), (K,))
    _same_gpu(what, Xc, W, smooth, inv_smooth)
    _check(lib().qv_smooth_calibrate(_ptr(Xc), _dtype(Xc), Mc, _ld(Xc), _ptr(W), _dtype(W), N, _ld(W), K,
                                     float(alpha), _ptr(smooth), _ptr(inv_smooth), _stream(stream)),
           "qv_smooth_calibrate")


# ------------------------------------------------------------------------------------------- W8A8

def qv_hadamard_smooth_quant8(X, inv_smooth, Xq8, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq8 [M, K] int8 codes, x_scale [M] fp32 (scale absmax / 127)."""
    M, K = _check_rotate_quant("qv_hadamard_smooth_quant8", X, inv_smooth, Xq8, x_scale, lambda K: K,
                               lambda M, K: (M,))
    _check(lib().qv_hadamard_smooth_quant8(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Xq8),
                                           _ptr(x_scale), _stream(stream)), "qv_hadamard_smooth_quant8")


def qv_pack_weights8(W, smooth, Wq8, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq8 [N, K] int8 codes, w_scale [N] fp32."""
    N, K = _check_rotate_quant("qv_pack_weights8", W, smooth, Wq8, w_scale, lambda K: K, lambda M, K: (M,))
    _check(lib().qv_pack_weights8(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), _ptr(Wq8), _ptr(w_scale),
                                  _stream(stream)), "qv_pack_weights8")


def qv_w8a8_gemm(Xq8, x_scale, Wq8, w_scale, bias, Y, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] (fp32/bf16) = dequant(Xq8 . Wq8^T) (+ bias) (+ GELU)."""
    M, N, K = _check_gemm("qv_w8a8_gemm", Xq8, x_scale, Wq8, w_scale, bias, Y, "int8", lambda c: c)
    _check(lib().qv_w8a8_gemm(_ptr(Xq8), _ptr(x_scale), _ptr(Wq8), _ptr(w_scale), _ptr(bias), M, N, K, int(epi),
                              _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)), "qv_w8a8_gemm")


def qv_w8a8_linear_workspace_size(M: int, K: int) -> int:
    return int(lib().qv_w8a8_linear_workspace_size(int(M), int(K)))


def qv_w8a8_linear(X, inv_smooth, Wq8, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE, stream=None) -> None:
    """The whole online W8A8 layer; ``workspace`` holds at least ``qv_w8a8_linear_workspace_size(M, K)`` bytes."""
    what = "qv_w8a8_linear"
    M, K = _rows_cols(what, "X", X)
    N = _rows_cols(what, "Wq8", Wq8)[0]
    _spec(what, "X", X, _FLOAT, (M, K), rows_packed=True)
    _spec(what, "inv_smooth", inv_smooth, ("float32",), (K,), optional=True)
    _spec(what, "Wq8", Wq8, ("int8",), (N, K))
    _spec(what, "w_scale", w_scale, ("float32",), (N,))
    _spec(what, "bias", bias, ("float32",), (N,), optional=True)
    _spec(what, "Y", Y, _FLOAT, (M, N), rows_packed=True)
    _check_workspace(what, workspace, qv_w8a8_linear_workspace_size(M, K))
    _same_gpu(what, X, inv_smooth, Wq8, w_scale, bias, Y, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w8a8_linear(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Wq8), _ptr(w_scale),
                                _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y), _ptr(workspace), nbytes,
                                _stream(stream)), "qv_w8a8_linear")


# -------------------------------------------------------------------------- group-wise granularity

def _group_count(what: str, K: int, group: int) -> int:
    if int(group) <= 0 or K % int(group):
        raise ValueError(f"{what}: group {group} must be positive and divide K = {K}")
    return K // int(group)


def qv_hadamard_smooth_quant_grouped(X, inv_smooth, group: int, Xq, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq [M, K/2] uint8 (packed int4), x_scale [M, K/group] fp32."""
    what = "qv_hadamard_smooth_quant_grouped"
    M, K = _check_rotate_quant(what, X, inv_smooth, Xq, x_scale, lambda K: K // 2,
                               lambda M, K: (M, _group_count(what, K, group)))
    _check(lib().qv_hadamard_smooth_quant_grouped(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), int(group),
                                                  _ptr(Xq), _ptr(x_scale), _stream(stream)),
           "qv_hadamard_smooth_quant_grouped")


def qv_pack_weights_grouped(W, smooth, group: int, Wq, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq [N, K/2] uint8 (packed int4), w_scale [N, K/group] fp32."""
    what = "qv_pack_weights_grouped"
    N, K = _check_rotate_quant(what, W, smooth, Wq, w_scale, lambda K: K // 2,
                               lambda M, K: (M, _group_count(what, K, group)))
    _check(lib().qv_pack_weights_grouped(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), int(group), _ptr(Wq),
                                         _ptr(w_scale), _stream(stream)), "qv_pack_weights_grouped")


def qv_w4a4_gemm_grouped(Xq, x_scale, Wq, w_scale, bias, Y, group: int, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] = sum over groups of dequantized int4 dot products (+ bias) (+ GELU)."""
    what = "qv_w4a4_gemm_grouped"
    M, N, K = _check_gemm(what, Xq, x_scale, Wq, w_scale, bias, Y, "uint8", lambda c: 2 * c,
                          lambda K: _group_count(what, K, group))
    _check(lib().qv_w4a4_gemm_grouped(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, K,
                                      int(group), int(epi), _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)),
           "qv_w4a4_gemm_grouped")


def qv_w4a4_linear_grouped_workspace_size(M: int, K: int, group: int) -> int:
    return int(lib().qv_w4a4_linear_grouped_workspace_size(int(M), int(K), int(group)))


def qv_w4a4_linear_grouped(X, inv_smooth, group: int, Wq, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE,
                           stream=None) -> None:
    """The whole online layer with group-wise scales; ``workspace`` holds at least
    ``qv_w4a4_linear_grouped_workspace_size(M, K, group)`` bytes."""
    what = "qv_w4a4_linear_grouped"
    M, K = _rows_cols(what, "X", X)
    N = _rows_cols(what, "Wq", Wq)[0]
    G = _group_count(what, K, group)
    _spec(what, "X", X, _FLOAT, (M, K), rows_packed=True)
    _spec(what, "inv_smooth", inv_smooth, ("float32",), (K,), optional=True)
    _spec(what, "Wq", Wq, ("uint8",), (N, K // 2))
    _spec(what, "w_scale", w_scale, ("float32",), (N, G))
    _spec(what, "bias", bias, ("float32",), (N,), optional=True)
    _spec(what, "Y", Y, _FLOAT, (M, N), rows_packed=True)
    _check_workspace(what, workspace, qv_w4a4_linear_grouped_workspace_size(M, K, group))
    _same_gpu(what, X, inv_smooth, Wq, w_scale, bias, Y, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w4a4_linear_grouped(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), int(group), _ptr(Wq),
                                        _ptr(w_scale), _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y),
                                        _ptr(workspace), nbytes, _stream(stream)), "qv_w4a4_linear_grouped")
