"""Acceptance rules of the parity tests (HIP path vs the oracle).

Codes.  The oracle rotates in fp64 and decides each code in fp32 from the correctly rounded rotated
value; the kernel sums the butterflies in fp32 and multiplies by the reciprocal of the scale.  The
two can disagree only where x / s lies within the kernel's rounding error of a half-integer.  For
every element this module bounds that error (first order, with a factor 2 of margin):
  * butterflies: each of the log2(K) stages rounds once, and the rounding errors feeding one output
    sum to at most log2(K) * u * sum_i |x_i| before the 1/sqrt(K) scaling (u = 2^-24).  Where the
    kernel forms the first five stages as one fp32 matrix-core sum of 32 exact products (bf16 rows
    of width 4096), that sum's error is measured below 3 u * sum |x| over its 32 terms, inside the
    5 u the five stages are allowed;
  * the smoothing product, the reciprocal of the scale and the fused rounding add a few u * |t|;
  * the row maximum, hence the scale, moves by at most the butterfly bound of its element.
A GPU code is admissible when it lies between rne(t - tau) and rne(t + tau), t the exact code-space
value; at most 1e-4 of all codes may differ from the oracle's.

Outputs.  Where a code differs the reference output is recomputed by the oracle from the GPU's own
codes and scales, so the output check isolates the contraction and the epilogue:
max |y - y_ref| / |y_ref| <= 1e-3 (0/0 counts as 0) for fp32 outputs, and for bf16 outputs the
GPU value must be within one bf16 ulp of y_ref rounded to bf16 (a bf16 ulp exceeds 1e-3).  Below the
fp32 normal range (|y_ref| < 2^-126) only an absolute difference of at most 2^-126 is required.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

U = 2.0 ** -24
FLT_MIN32 = np.float32(2.0 ** -126)
CODE_MISMATCH_MAX = 1e-4
OUT_REL_MAX = 1e-3


def code_bounds(X, mult, Xhat=None, dX=None, qmax: int = 7):
    """Exact code-space values t and the per-element tolerance tau for rows X (fp32 values).

    ``dX`` (optional, same shape) bounds how far the GPU's input rows may differ from X elementwise
    (a chained layer fed the GPU's previous output): each rotated element then moves by at most
    sum_i |dX_i| / sqrt(K) more, since every entry of H / sqrt(K) is +-1/sqrt(K)."""
    X = np.asarray(X, dtype=np.float64)
    M, K = X.shape
    if Xhat is None:
        Xhat = oracle.rotate(X, oracle.ROT_FWHT)
    m = np.ones(K) if mult is None else np.asarray(mult, dtype=np.float64)
    L = math.log2(K)
    xt = Xhat * m
    a = np.max(np.abs(xt), axis=1)
    s = a / float(qmax)
    # Rows whose fp32 scale is zero or subnormal quantize to all-zero codes on both sides.
    flushed = (np.max(np.abs(Xhat.astype(np.float32) * m.astype(np.float32)), axis=1) / np.float32(qmax)) < FLT_MIN32
    s = np.where(flushed, 0.0, s)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, None] > 0, xt / s[:, None], 0.0)
        e_x = L * U * np.sum(np.abs(X), axis=1) / math.sqrt(K)  # butterfly error bound per row
        if dX is not None:
            d1 = np.sum(np.abs(np.asarray(dX, dtype=np.float64)), axis=1) / math.sqrt(K)
            e_x = e_x + L * U * d1 + d1
        rel_scale = np.where(a > 0, e_x * np.max(np.abs(m)) / a, 0.0) + 4 * U
        tau = 2.0 * ((e_x[:, None] * np.abs(m)[None, :] + 2 * U * np.abs(xt)) / np.where(s > 0, s, 1.0)[:, None]
                     + np.abs(t) * rel_scale[:, None])
    return t, tau, s, rel_scale


def check_codes(q_gpu, q_ref, t, tau, label="", qmax: int = 7):
    """Every GPU code admissible; mismatch rate <= 1e-4.  Returns the mismatch rate."""
    q_gpu = np.asarray(q_gpu, dtype=np.int64)
    q_ref = np.asarray(q_ref, dtype=np.int64)
    lo = np.clip(np.rint(t - tau), -qmax - 1, qmax)
    hi = np.clip(np.rint(t + tau), -qmax - 1, qmax)
    bad = (q_gpu < lo) | (q_gpu > hi)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), int(q_gpu[tuple(i)]), int(q_ref[tuple(i)]), float(t[tuple(i)]), float(tau[tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{label}: {int(bad.sum())} inadmissible codes, e.g. (idx, gpu, ref, t, tau) {detail}")
    rate = float(np.mean(q_gpu != q_ref)) if q_ref.size else 0.0
    assert rate <= CODE_MISMATCH_MAX, f"{label}: code mismatch rate {rate:.2e} > {CODE_MISMATCH_MAX}"
    return rate


def check_scales(s_gpu, s_ref, rel_scale, label=""):
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    tol = 2.0 * rel_scale * np.abs(s_ref) + 1e-45
    bad = np.abs(s_gpu - s_ref) > tol
    assert not np.any(bad), f"{label}: {int(bad.sum())} scales out of tolerance, first {np.argwhere(bad)[:3].ravel()}"


def bf16_round(y):
    """fp64 -> nearest bf16 (ties to even) as fp64, through fp32 first as the kernel does."""
    f = np.asarray(y, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


BF16_SUBNORMAL_STEP = 2.0 ** -133


def bf16_ulp(r):
    """The spacing of bf16 values in the binade of r: 2^(floor(log2 |r|) - 7) for normal r (8
    significant bits), and the subnormal step 2^-133 below the normal range and at zero."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    _, e = np.frexp(r)  # r = f * 2^e with f in [0.5, 1), so floor(log2 r) = e - 1 (frexp(0) gives e = 0)
    return np.where(r > 0, np.maximum(np.ldexp(1.0, e - 8), BF16_SUBNORMAL_STEP), BF16_SUBNORMAL_STEP)


def check_outputs(y_gpu, y_ref, out_bf16: bool, label=""):
    """Returns the worst relative error (fp32 outputs) or the worst difference in bf16 ulps."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if out_bf16:
        r = bf16_round(y_ref)
        ulp = bf16_ulp(r)
        bad = np.abs(y_gpu - r) > ulp
        assert not np.any(bad), (f"{label}: {int(bad.sum())} bf16 outputs beyond 1 ulp, e.g. "
                                 f"{[(float(y_gpu[tuple(i)]), float(y_ref[tuple(i)])) for i in np.argwhere(bad)[:3]]}")
        # Reported: the largest difference from the rounded reference, in bf16 ulps at its magnitude.
        with np.errstate(divide="ignore", invalid="ignore"):
            ulps = np.where(np.abs(y_gpu - r) > 0, np.abs(y_gpu - r) / ulp, 0.0)
        return float(np.max(ulps)) if y_ref.size else 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.abs(y_gpu - y_ref) / np.abs(y_ref)
    rel[(y_gpu == y_ref)] = 0.0
    # Below the fp32 normal range (e.g. the far negative GELU tail) an fp32 output cannot carry a
    # relative accuracy; there the absolute difference must stay below the smallest normal.
    tiny = np.abs(y_ref) < float(FLT_MIN32)
    rel[tiny] = np.where(np.abs(y_gpu[tiny] - y_ref[tiny]) <= float(FLT_MIN32), 0.0, np.inf)
    worst = float(np.max(rel)) if rel.size else 0.0
    assert worst <= OUT_REL_MAX, f"{label}: max relative error {worst:.3e} > {OUT_REL_MAX}"
    return worst


# ------------------------------------------------------------------ group-wise granularity
# The same bounds with one scale per row and group of channels: the butterfly error of an element
# is the row's (the rotation is over the whole row), the scale is its group's.

def code_bounds_grouped(X, mult, group: int, Xhat=None, qmax: int = 7):
    """t, tau (as code_bounds) and the per-(row, group) scales and relative scale tolerances."""
    X = np.asarray(X, dtype=np.float64)
    M, K = X.shape
    G = K // group
    if Xhat is None:
        Xhat = oracle.rotate(X, oracle.ROT_FWHT)
    m = np.ones(K) if mult is None else np.asarray(mult, dtype=np.float64)
    L = math.log2(K)
    xt = Xhat * m
    a = np.max(np.abs(xt).reshape(M, G, group), axis=2)
    flushed = (np.max(np.abs(Xhat.astype(np.float32) * m.astype(np.float32)).reshape(M, G, group), axis=2)
               / np.float32(qmax)) < FLT_MIN32
    s = np.where(flushed, 0.0, a / float(qmax))
    se = np.repeat(s, group, axis=1)
    mmax = np.max(np.abs(m).reshape(G, group), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(se > 0, xt / se, 0.0)
        e_x = L * U * np.sum(np.abs(X), axis=1) / math.sqrt(K)
        rel_scale = np.where(a > 0, e_x[:, None] * mmax[None, :] / a, 0.0) + 4 * U
        tau = 2.0 * ((e_x[:, None] * np.abs(m)[None, :] + 2 * U * np.abs(xt)) / np.where(se > 0, se, 1.0)
                     + np.abs(t) * np.repeat(rel_scale, group, axis=1))
    return t, tau, s, rel_scale


def grouped_abs_sum(qa, qw, sa, sw):
    """sum_g |acc_g| sa[:, g] sw[:, g] (fp64) from int8 codes: the size of the terms the fp32
    accumulation of a grouped product adds up."""
    qa = np.asarray(qa, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    K = qa.shape[1]
    G = sa.shape[1]
    group = K // G
    out = np.zeros((qa.shape[0], qw.shape[0]))
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        acc = oracle.gemm_int(qa[:, sl], qw[:, sl]).astype(np.float64)
        out += np.abs(acc) * sa[:, g:g + 1].astype(np.float64) * sw[:, g].astype(np.float64)[None, :]
    return out


def check_outputs_grouped(y_gpu, y_ref, y_abs, out_bf16: bool, groups: int, label=""):
    """Grouped outputs: each group adds one product and one fp32 sum to the accumulator, so beyond
    the relative bar of check_outputs an absolute (groups + 3) * 2u * sum_g |term_g| is allowed
    (x 1.2 for the GELU's slope).  Returns the worst error in units of the allowance."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    extra = 1.2 * 2.0 * (groups + 3) * U * np.asarray(y_abs, dtype=np.float64)
    if out_bf16:
        r = bf16_round(y_ref)
        allow = bf16_ulp(r) + extra
        err = np.abs(y_gpu - r)
    else:
        allow = OUT_REL_MAX * np.abs(y_ref) + extra + float(FLT_MIN32)
        err = np.abs(y_gpu - y_ref)
    bad = err > allow
    assert not np.any(bad), (f"{label}: {int(bad.sum())} outputs beyond the bound, e.g. "
                             f"{[(float(y_gpu[tuple(i)]), float(y_ref[tuple(i)])) for i in np.argwhere(bad)[:3]]}")
    return float(np.max(err / allow)) if err.size else 0.0
