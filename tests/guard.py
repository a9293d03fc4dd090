"""Output buffers with guard space for the GEMM tests.

The output is a view of the first M rows and N columns of a larger NaN-filled buffer: GUARD_ROWS
more rows (more than a row tile) and the row padding.  After a launch every element outside the
view must still be NaN, so a store past the last row or column of a ragged tile is caught."""
import torch

GUARD_ROWS = 256


def guarded_output(M, N, dtype, dev, ldy_pad=0):
    """(full buffer, the [M, N] output view with row stride N + ldy_pad)."""
    full = torch.full((M + GUARD_ROWS, N + ldy_pad), float("nan"), dtype=dtype, device=dev)
    return full, full[:M, :N]


def check_guard(full, M, N, label=""):
    rows_ok = bool(torch.isnan(full[M:].float()).all())
    cols_ok = bool(torch.isnan(full[:M, N:].float()).all()) if full.shape[1] > N else True
    assert rows_ok, f"{label}: wrote past the last output row"
    assert cols_ok, f"{label}: wrote outside the output columns"


def guarded_codes(M, row_bytes, n_scales, dev, code_dtype=torch.uint8, code_fill=0xAB):
    """(codes buffer, codes view [M, row_bytes], scales buffer, scales view) with GUARD_ROWS extra
    rows of fill (codes) and -1 (scales) after the views."""
    q = torch.full((M + GUARD_ROWS, row_bytes), code_fill, dtype=code_dtype, device=dev)
    shape = (M + GUARD_ROWS,) if n_scales == 0 else (M + GUARD_ROWS, n_scales)
    s = torch.full(shape, -1.0, dtype=torch.float32, device=dev)
    return q, q[:M], s, s[:M]


def check_codes_guard(q, s, M, code_fill=0xAB, label=""):
    assert bool((q[M:] == code_fill).all()), f"{label}: wrote codes past the last row"
    assert bool((s[M:] == -1.0).all()), f"{label}: wrote scales past the last row"
