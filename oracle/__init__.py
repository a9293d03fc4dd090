"""ctypes wrapper around the plain C oracle ``oracle/libqvref.so``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  Every function returns fresh numpy
arrays; inputs are converted to the C types the oracle takes (fp64 values, fp32 vectors, int8
codes), and those conversions are exact for fp32/bf16 inputs.

Sources are cited by page title and section (see ``qvref.h`` for the list):
``[P4]`` is the gslzct.com translation of the QuantVGGT method ("十亿参数的三维重建模型，能塞进手机吗？").
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QVREF_LIB points the wrapper at another build of the oracle (the mutation tests use it).
LIB_PATH = os.environ.get("QVREF_LIB") or os.path.join(_HERE, "libqvref.so")

ROT_EXPLICIT = 0
ROT_FWHT = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile ``qvref.c`` into ``libqvref.so`` with gcc (no intrinsics, no fast-math)."""
    from .build import build_oracle

    return build_oracle(force=force)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        P = ctypes.c_void_p
        sigs = {
            "qvref_hadamard_closed_form": [i64, P],
            "qvref_hadamard_sylvester": [i64, P],
            "qvref_rotate_explicit": [P, i64, i64, i64, P],
            "qvref_rotate_fwht": [P, i64, i64, i64, P],
            "qvref_quantize_rows": [P, i64, i64, P, i32, P, P],
            "qvref_pack_int4": [P, i64, i64, P],
            "qvref_unpack_int4": [P, i64, i64, P],
            "qvref_gemm_int": [P, P, i64, i64, i64, P],
            "qvref_dequant": [P, P, P, P, i64, i64, i32, P],
            "qvref_smoothing": [P, i64, P, i64, i64, dbl, P, P],
            "qvref_hadamard_smooth_quant": [P, i64, i64, i64, P, i32, P, P],
            "qvref_pack_weights": [P, i64, i64, i64, P, i32, P, P],
            "qvref_w4a4_gemm": [P, P, P, P, P, i64, i64, i64, i32, P, P],
            "qvref_w4a4_linear": [P, i64, i64, i64, P, P, P, P, i64, i32, i32, P],
            "qvref_dequant_grouped": [P, P, P, P, P, i64, i64, i64, i64, i32, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.qvref_gelu.argtypes = [dbl]
        L.qvref_gelu.restype = dbl
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _f32(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _check(rc, what):
    if rc == -2:
        raise OverflowError(f"{what}: int32 accumulator overflow")
    if rc != 0:
        raise ValueError(f"{what}: bad arguments (rc={rc})")


def hadamard(d: int, method: str = "closed_form") -> np.ndarray:
    H = np.empty((d, d), dtype=np.int8)
    fn = lib().qvref_hadamard_closed_form if method == "closed_form" else lib().qvref_hadamard_sylvester
    _check(fn(d, _p(H)), "hadamard")
    return H


def rotate(X, mode: int = ROT_EXPLICIT) -> np.ndarray:
    """Rows of X times H_d / sqrt(d), fp64 ([P4] 预全局旋转)."""
    X = _f64(X)
    M, d = X.shape
    Y = np.empty((M, d), dtype=np.float64)
    fn = lib().qvref_rotate_explicit if mode == ROT_EXPLICIT else lib().qvref_rotate_fwht
    _check(fn(_p(X), M, d, d, _p(Y)), "rotate")
    return Y


def quantize_rows(Xhat, mult=None, bits: int = 4):
    """Symmetric per-row quantization of rotated rows ([P4] 训练后量化（PTQ）); returns (q, scale)."""
    Xhat = _f64(Xhat)
    M, K = Xhat.shape
    mult = _f32(mult)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    _check(lib().qvref_quantize_rows(_p(Xhat), M, K, _p(mult), bits, _p(q), _p(s)), "quantize_rows")
    return q, s


def pack_int4(q) -> np.ndarray:
    q = np.ascontiguousarray(np.asarray(q, dtype=np.int8))
    R, K = q.shape
    out = np.empty((R, K // 2), dtype=np.uint8)
    _check(lib().qvref_pack_int4(_p(q), R, K, _p(out)), "pack_int4")
    return out


def unpack_int4(packed) -> np.ndarray:
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    R, Kh = packed.shape
    q = np.empty((R, 2 * Kh), dtype=np.int8)
    _check(lib().qvref_unpack_int4(_p(packed), R, 2 * Kh, _p(q)), "unpack_int4")
    return q


def gemm_int(qa, qw) -> np.ndarray:
    """acc = qa . qw^T exactly (int64 accumulation, int32 result)."""
    qa = np.ascontiguousarray(np.asarray(qa, dtype=np.int8))
    qw = np.ascontiguousarray(np.asarray(qw, dtype=np.int8))
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib().qvref_gemm_int(_p(qa), _p(qw), M, N, K, _p(acc)), "gemm_int")
    return acc


def dequant(acc, sa, sw, bias=None, epi: int = 0) -> np.ndarray:
    acc = np.ascontiguousarray(np.asarray(acc, dtype=np.int32))
    M, N = acc.shape
    sa, sw, bias = _f32(sa), _f32(sw), _f32(bias)
    Y = np.empty((M, N), dtype=np.float64)
    _check(lib().qvref_dequant(_p(acc), _p(sa), _p(sw), _p(bias), M, N, epi, _p(Y)), "dequant")
    return Y


def gelu(y: float) -> float:
    return lib().qvref_gelu(float(y))


def smoothing(Xhat_calib, What, alpha: float = 0.5):
    """Per-channel smoothing factors from rotated statistics ([P4] 后局部平滑); returns (s, 1/s)."""
    Xh = _f64(Xhat_calib)
    Wh = _f64(What)
    Mc, K = Xh.shape
    N = Wh.shape[0]
    s = np.empty((K,), dtype=np.float32)
    inv = np.empty((K,), dtype=np.float32)
    _check(lib().qvref_smoothing(_p(Xh), Mc, _p(Wh), N, K, float(alpha), _p(s), _p(inv)), "smoothing")
    return s, inv


def hadamard_smooth_quant(X, inv_smooth=None, mode: int = ROT_EXPLICIT):
    """Oracle of the activation step: returns (Xq packed [M, K/2] uint8, x_scale [M] fp32)."""
    X = _f64(X)
    M, K = X.shape
    inv_smooth = _f32(inv_smooth)
    Xq = np.empty((M, K // 2), dtype=np.uint8)
    xs = np.empty((M,), dtype=np.float32)
    _check(lib().qvref_hadamard_smooth_quant(_p(X), M, K, K, _p(inv_smooth), mode, _p(Xq), _p(xs)),
           "hadamard_smooth_quant")
    return Xq, xs


def pack_weights(W, smooth=None, mode: int = ROT_EXPLICIT):
    """Oracle of the offline weight step: returns (Wq packed [N, K/2] uint8, w_scale [N] fp32)."""
    W = _f64(W)
    N, K = W.shape
    smooth = _f32(smooth)
    Wq = np.empty((N, K // 2), dtype=np.uint8)
    ws = np.empty((N,), dtype=np.float32)
    _check(lib().qvref_pack_weights(_p(W), N, K, K, _p(smooth), mode, _p(Wq), _p(ws)), "pack_weights")
    return Wq, ws


def w4a4_gemm(Xq, x_scale, Wq, w_scale, bias=None, epi: int = 0, return_acc: bool = False):
    Xq = np.ascontiguousarray(np.asarray(Xq, dtype=np.uint8))
    Wq = np.ascontiguousarray(np.asarray(Wq, dtype=np.uint8))
    M, Kh = Xq.shape
    N = Wq.shape[0]
    xs, ws, bias = _f32(x_scale), _f32(w_scale), _f32(bias)
    Y = np.empty((M, N), dtype=np.float64)
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib().qvref_w4a4_gemm(_p(Xq), _p(xs), _p(Wq), _p(ws), _p(bias), M, N, 2 * Kh, epi, _p(Y),
                                 _p(acc)), "w4a4_gemm")
    return (Y, acc) if return_acc else Y


def w4a4_linear(X, inv_smooth, Wq, w_scale, bias=None, epi: int = 0, mode: int = ROT_EXPLICIT):
    X = _f64(X)
    M, K = X.shape
    Wq = np.ascontiguousarray(np.asarray(Wq, dtype=np.uint8))
    N = Wq.shape[0]
    inv_smooth, ws, bias = _f32(inv_smooth), _f32(w_scale), _f32(bias)
    Y = np.empty((M, N), dtype=np.float64)
    _check(lib().qvref_w4a4_linear(_p(X), M, K, K, _p(inv_smooth), _p(Wq), _p(ws), _p(bias), N, epi,
                                   mode, _p(Y)), "w4a4_linear")
    return Y


# ---------------------------------------------------------------- W8A8 ([P4] 训练后量化（PTQ）, N = 8)
# The pages' second setting: the same rotation and smoothing, codes in [-128, 127] with scale
# absmax / 127, one int8 code per element (no packing).  Composed from the primitives above.

def hadamard_smooth_quant8(X, inv_smooth=None, mode: int = ROT_EXPLICIT):
    """Oracle of the 8-bit activation step: returns (Xq8 [M, K] int8, x_scale [M] fp32)."""
    return quantize_rows(rotate(X, mode), inv_smooth, bits=8)


def pack_weights8(W, smooth=None, mode: int = ROT_EXPLICIT):
    """Oracle of the 8-bit weight step: returns (Wq8 [N, K] int8, w_scale [N] fp32)."""
    return quantize_rows(rotate(W, mode), smooth, bits=8)


def w8a8_gemm(Xq8, x_scale, Wq8, w_scale, bias=None, epi: int = 0, return_acc: bool = False):
    """acc = Xq8 . Wq8^T (exact), Y = dequant(acc) (+ bias) (+ GELU)."""
    acc = gemm_int(Xq8, Wq8)
    Y = dequant(acc, x_scale, w_scale, bias, epi)
    return (Y, acc) if return_acc else Y


# ------------------------------------------------ group-wise granularity ([P4] 细粒度量化粒度)
# The subsection is truncated on the page.  Reading: the rotation and smoothing stay as above
# (pre-global, over the whole row); each row of activations and of weights is then quantized in
# groups of `group` consecutive channels, each group with its own symmetric scale absmax / 7, and
# the product sums the groups' integer dot products dequantized by their own pair of scales.
# The quantizer is the per-row one applied to each group's slice of the row.

def quantize_groups(Xhat, mult=None, group: int = 128, bits: int = 4):
    """Symmetric quantization per (row, group of channels); returns (q [R, K], scale [R, K/group])."""
    Xhat = _f64(Xhat)
    R, K = Xhat.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    mult = None if mult is None else np.asarray(mult, dtype=np.float32)
    q = np.empty((R, K), dtype=np.int8)
    s = np.empty((R, K // group), dtype=np.float32)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        q[:, sl], s[:, g] = quantize_rows(Xhat[:, sl], None if mult is None else mult[sl], bits)
    return q, s


def hadamard_smooth_quant_grouped(X, inv_smooth=None, group: int = 128, mode: int = ROT_EXPLICIT):
    """Grouped activation step: returns (Xq packed [M, K/2] uint8, x_scale [M, K/group] fp32)."""
    q, s = quantize_groups(rotate(X, mode), inv_smooth, group)
    return pack_int4(q), s


def pack_weights_grouped(W, smooth=None, group: int = 128, mode: int = ROT_EXPLICIT):
    """Grouped weight step: returns (Wq packed [N, K/2] uint8, w_scale [N, K/group] fp32)."""
    q, s = quantize_groups(rotate(W, mode), smooth, group)
    return pack_int4(q), s


def dequant_grouped(qa, qw, sa, sw, bias=None, epi: int = 0) -> np.ndarray:
    """Y = sum_g acc_g * sa[:, g] * sw[:, g] (+ bias) (+ GELU) in fp64 from int8 codes."""
    qa = np.ascontiguousarray(np.asarray(qa, dtype=np.int8))
    qw = np.ascontiguousarray(np.asarray(qw, dtype=np.int8))
    M, K = qa.shape
    N = qw.shape[0]
    sa = np.ascontiguousarray(np.asarray(sa, dtype=np.float32))
    sw = np.ascontiguousarray(np.asarray(sw, dtype=np.float32))
    group = K // sa.shape[1]
    Y = np.empty((M, N), dtype=np.float64)
    bias = _f32(bias)
    _check(lib().qvref_dequant_grouped(_p(qa), _p(qw), _p(sa), _p(sw), _p(bias), M, N, K, group, epi,
                                       _p(Y)), "dequant_grouped")
    return Y


def w4a4_gemm_grouped(Xq, x_scale, Wq, w_scale, bias=None, epi: int = 0) -> np.ndarray:
    """Grouped GEMM on packed codes: unpack, then dequant_grouped."""
    return dequant_grouped(unpack_int4(Xq), unpack_int4(Wq), x_scale, w_scale, bias, epi)
