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
    "qv_w4a4_linear_workspace_size", "qv_w4a4_linear", "qv_smooth_calibrate",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libqv.so")

QV_F32, QV_BF16 = 0, 1
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
        L = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.qv_status_string.argtypes = [i32]
        L.qv_status_string.restype = ctypes.c_char_p
        L.qv_hadamard_smooth_quant.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
        L.qv_pack_weights.argtypes = [P, i32, i64, i64, i64, P, P, P, P]
        L.qv_w4a4_gemm.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P, i32, i64, P]
        L.qv_w4a4_linear_workspace_size.argtypes = [i64, i64]
        L.qv_w4a4_linear_workspace_size.restype = sz
        L.qv_w4a4_linear.argtypes = [P, i32, i64, i64, i64, P, P, P, P, i64, i32, P, i32, i64, P, sz, P]
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
                     "qv_smooth_calibrate", "qv_hadamard_smooth_quant8", "qv_pack_weights8", "qv_w8a8_gemm",
                     "qv_w8a8_linear", "qv_hadamard_smooth_quant_grouped", "qv_pack_weights_grouped",
                     "qv_w4a4_gemm_grouped", "qv_w4a4_linear_grouped"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


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
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def qv_hadamard_smooth_quant(X, inv_smooth, Xq, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq [M, K/2] uint8 (packed int4), x_scale [M] fp32."""
    M, K = X.shape
    _check(lib().qv_hadamard_smooth_quant(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Xq),
                                          _ptr(x_scale), _stream(stream)), "qv_hadamard_smooth_quant")


def qv_pack_weights(W, smooth, Wq, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq [N, K/2] uint8 (packed int4), w_scale [N] fp32."""
    N, K = W.shape
    _check(lib().qv_pack_weights(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), _ptr(Wq), _ptr(w_scale),
                                 _stream(stream)), "qv_pack_weights")


def qv_w4a4_gemm(Xq, x_scale, Wq, w_scale, bias, Y, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] (fp32/bf16) = dequant(Xq . Wq^T) (+ bias) (+ GELU)."""
    M, Kh = Xq.shape
    N = Wq.shape[0]
    _check(lib().qv_w4a4_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, 2 * Kh, int(epi),
                              _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)), "qv_w4a4_gemm")


def qv_w4a4_linear_workspace_size(M: int, K: int) -> int:
    return int(lib().qv_w4a4_linear_workspace_size(int(M), int(K)))


def qv_w4a4_linear(X, inv_smooth, Wq, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE, stream=None) -> None:
    """The whole online layer; ``workspace`` is a uint8 device tensor of at least
    ``qv_w4a4_linear_workspace_size(M, K)`` bytes."""
    M, K = X.shape
    N = Wq.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w4a4_linear(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Wq), _ptr(w_scale),
                                _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y), _ptr(workspace), nbytes,
                                _stream(stream)), "qv_w4a4_linear")


def qv_smooth_calibrate(Xc, W, smooth, inv_smooth, alpha: float = 0.5, stream=None) -> None:
    """smooth [K], inv_smooth [K] fp32 from the rotated calibration rows Xc [Mc, K] and weights W [N, K]."""
    Mc, K = Xc.shape
    N = W.shape[0]
    _check(lib().qv_smooth_calibrate(_ptr(Xc), _dtype(Xc), Mc, _ld(Xc), _ptr(W), _dtype(W), N, _ld(W), K,
                                     float(alpha), _ptr(smooth), _ptr(inv_smooth), _stream(stream)),
           "qv_smooth_calibrate")


# ------------------------------------------------------------------------------------------- W8A8

def qv_hadamard_smooth_quant8(X, inv_smooth, Xq8, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq8 [M, K] int8 codes, x_scale [M] fp32 (scale absmax / 127)."""
    M, K = X.shape
    _check(lib().qv_hadamard_smooth_quant8(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Xq8),
                                           _ptr(x_scale), _stream(stream)), "qv_hadamard_smooth_quant8")


def qv_pack_weights8(W, smooth, Wq8, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq8 [N, K] int8 codes, w_scale [N] fp32."""
    N, K = W.shape
    _check(lib().qv_pack_weights8(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), _ptr(Wq8), _ptr(w_scale),
                                  _stream(stream)), "qv_pack_weights8")


def qv_w8a8_gemm(Xq8, x_scale, Wq8, w_scale, bias, Y, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] (fp32/bf16) = dequant(Xq8 . Wq8^T) (+ bias) (+ GELU)."""
    M, K = Xq8.shape
    N = Wq8.shape[0]
    _check(lib().qv_w8a8_gemm(_ptr(Xq8), _ptr(x_scale), _ptr(Wq8), _ptr(w_scale), _ptr(bias), M, N, K, int(epi),
                              _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)), "qv_w8a8_gemm")


def qv_w8a8_linear_workspace_size(M: int, K: int) -> int:
    return int(lib().qv_w8a8_linear_workspace_size(int(M), int(K)))


def qv_w8a8_linear(X, inv_smooth, Wq8, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE, stream=None) -> None:
    """The whole online W8A8 layer; ``workspace`` holds at least ``qv_w8a8_linear_workspace_size(M, K)`` bytes."""
    M, K = X.shape
    N = Wq8.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w8a8_linear(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), _ptr(Wq8), _ptr(w_scale),
                                _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y), _ptr(workspace), nbytes,
                                _stream(stream)), "qv_w8a8_linear")


# -------------------------------------------------------------------------- group-wise granularity

def _group_scales(scale, rows: int, K: int, group: int) -> None:
    if tuple(scale.shape) != (rows, K // group) or not scale.is_contiguous():
        raise ValueError(f"group scales must be a contiguous [{rows}, {K // group}] tensor")


def qv_hadamard_smooth_quant_grouped(X, inv_smooth, group: int, Xq, x_scale, stream=None) -> None:
    """X [M, K] fp32/bf16 -> Xq [M, K/2] uint8 (packed int4), x_scale [M, K/group] fp32."""
    M, K = X.shape
    _group_scales(x_scale, M, K, group)
    _check(lib().qv_hadamard_smooth_quant_grouped(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), int(group),
                                                  _ptr(Xq), _ptr(x_scale), _stream(stream)),
           "qv_hadamard_smooth_quant_grouped")


def qv_pack_weights_grouped(W, smooth, group: int, Wq, w_scale, stream=None) -> None:
    """W [N, K] fp32/bf16 -> Wq [N, K/2] uint8 (packed int4), w_scale [N, K/group] fp32."""
    N, K = W.shape
    _group_scales(w_scale, N, K, group)
    _check(lib().qv_pack_weights_grouped(_ptr(W), _dtype(W), N, K, _ld(W), _ptr(smooth), int(group), _ptr(Wq),
                                         _ptr(w_scale), _stream(stream)), "qv_pack_weights_grouped")


def qv_w4a4_gemm_grouped(Xq, x_scale, Wq, w_scale, bias, Y, group: int, epi: int = QV_EPI_NONE, stream=None) -> None:
    """Y [M, N] = sum over groups of dequantized int4 dot products (+ bias) (+ GELU)."""
    M, Kh = Xq.shape
    N = Wq.shape[0]
    _group_scales(x_scale, M, 2 * Kh, group)
    _group_scales(w_scale, N, 2 * Kh, group)
    _check(lib().qv_w4a4_gemm_grouped(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(bias), M, N, 2 * Kh,
                                      int(group), int(epi), _ptr(Y), _dtype(Y), _ld(Y), _stream(stream)),
           "qv_w4a4_gemm_grouped")


def qv_w4a4_linear_grouped_workspace_size(M: int, K: int, group: int) -> int:
    return int(lib().qv_w4a4_linear_grouped_workspace_size(int(M), int(K), int(group)))


def qv_w4a4_linear_grouped(X, inv_smooth, group: int, Wq, w_scale, bias, Y, workspace, epi: int = QV_EPI_NONE,
                           stream=None) -> None:
    """The whole online layer with group-wise scales; ``workspace`` holds at least
    ``qv_w4a4_linear_grouped_workspace_size(M, K, group)`` bytes."""
    M, K = X.shape
    N = Wq.shape[0]
    _group_scales(w_scale, N, K, group)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qv_w4a4_linear_grouped(_ptr(X), _dtype(X), M, K, _ld(X), _ptr(inv_smooth), int(group), _ptr(Wq),
                                        _ptr(w_scale), _ptr(bias), N, int(epi), _ptr(Y), _dtype(Y), _ld(Y),
                                        _ptr(workspace), nbytes, _stream(stream)), "qv_w4a4_linear_grouped")
