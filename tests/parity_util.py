"""Whole-output parity helpers shared by the GPU tests (test infrastructure).

The oracle's reference output is computed over every output row, in row chunks
so that the host holds at most `chunk` decoded rows at a time, and the GPU
result is compared with it in full: the global bar (relative L2 <= 1e-3, max
abs <= 1e-2 * max|y_ref|) over all outputs, and the same relative-L2 test per
block of 64 output rows with three times the global bound.  The per-block test
catches a fault confined to one workgroup's rows (a tile of 16 or 64 rows
with, say, a 1 % error would pass the global relative L2 of a 4096-row layer).
"""
import numpy as np

from oracle import aqlm_oracle as O

REL_L2 = 1e-3
MAX_ABS_FRAC = 1e-2
BLOCK_ROWS = 64
BLOCK_REL_L2 = 3 * REL_L2


def ref_full(L, x=None, chunk=2048):
    """y_ref [T][out] float64 over every row of layer L (codes, codebooks, scales)."""
    x = L.x if x is None else x
    out = L.codes.shape[0]
    parts = [O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, x, np.arange(r, min(r + chunk, out)))
             for r in range(0, out, chunk)]
    return np.concatenate(parts, axis=1)


def assert_close_all(y, y_ref, what=""):
    """Global bar over every output, then the per-64-row-block relative L2."""
    y = np.asarray(y, dtype=np.float64)
    rel, mx, ref_max = O.parity_errors(y, y_ref)
    assert np.isfinite(rel) and np.isfinite(y).all(), f"{what}: non-finite output"
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC * ref_max, f"{what}: max abs {mx:.3e} > 1e-2 * {ref_max:.3e}"
    out = y_ref.shape[1]
    for r0 in range(0, out, BLOCK_ROWS):
        a, b = y[:, r0:r0 + BLOCK_ROWS], y_ref[:, r0:r0 + BLOCK_ROWS]
        nb = float(np.linalg.norm(b))
        if nb == 0.0:
            assert not a.any(), f"{what}: rows {r0}+ should be zero"
            continue
        rb = float(np.linalg.norm(a - b)) / nb
        assert rb <= BLOCK_REL_L2, f"{what}: rows {r0}..{r0 + BLOCK_ROWS - 1} rel L2 {rb:.3e} > {BLOCK_REL_L2}"


def decode_full_bits(L, chunk=4096):
    """The oracle's fp16 decode of every row, as uint16 bit patterns."""
    out = L.codes.shape[0]
    return np.concatenate([O.decode_fp16(L.codes, L.codebooks, L.scales, rows=np.arange(r, min(r + chunk, out)))
                           .view(np.uint16) for r in range(0, out, chunk)])
