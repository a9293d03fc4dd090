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
