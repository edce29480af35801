"""Reference of the slice-list layout that aqlm_lists_plan / aqlm_lists_fill write.

Written from the layout's definition in include/aqlm.h (an integer regrouping of
the codes, no arithmetic of the method), in plain numpy, so that the library's
table and entries can be compared with it byte for byte.  Test infrastructure.
"""
from __future__ import annotations

import numpy as np

SLICES = 8
SLICE_BITS = 13
MAX_BLOCK = 1024


def geometry(out: int, n_in: int):
    """(G, J, Gb, Z, n_rt): groups per row, blocks, groups per block, zero chunk, row tiles."""
    G = n_in // 8
    J = -(-G // MAX_BLOCK)
    Gb = -(-G // J)
    Z = -(-Gb // 64) * 64
    n_rt = -(-out // 64)
    return G, J, Gb, Z, n_rt


def pack(codes: np.ndarray, n_in: int):
    """codes [out][in/8][1] int16 -> (table uint32 [2 n_units + 2], entries uint32 [steps * 64])."""
    c = codes.reshape(codes.shape[0], -1).view(np.uint16).astype(np.int64)
    out = c.shape[0]
    G, J, Gb, Z, n_rt = geometry(out, n_in)
    n_units = SLICES * J * n_rt
    table = np.zeros(2 * n_units + 2, np.uint32)
    pad = np.uint32(Z << SLICE_BITS)
    blocks = []
    off = 0
    for s in range(SLICES):
        for k in range(J):
            j0, j1 = k * Gb, min(G, (k + 1) * Gb)
            for rt in range(n_rt):
                rows = c[rt * 64: min(out, rt * 64 + 64), j0:j1]
                r, j = np.nonzero((rows >> SLICE_BITS) == s)        # row-major: ascending j within a row
                counts = np.bincount(r, minlength=64)
                L = int(counts.max()) if r.size else 0
                start = np.concatenate([[0], np.cumsum(counts)[:-1]])
                t = np.arange(r.size) - start[r]
                block = np.full((L, 64), pad, np.uint32)
                block[t, r] = ((j << SLICE_BITS) | (rows[r, j] & ((1 << SLICE_BITS) - 1))).astype(np.uint32)
                u = (s * J + k) * n_rt + rt
                table[2 * u] = off
                table[2 * u + 1] = L
                blocks.append(block.ravel())
                off += L
    table[2 * n_units: 2 * n_units + 2] = np.array([off], np.uint64).view(np.uint32)
    entries = np.concatenate(blocks) if blocks else np.zeros(0, np.uint32)
    return table, entries


def unpack(table: np.ndarray, entries: np.ndarray, out: int, n_in: int) -> np.ndarray:
    """Inverse of pack on the listed (non-padding) entries: codes [out][in/8][1] int16."""
    G, J, Gb, Z, n_rt = geometry(out, n_in)
    codes = np.full((out, G), -1, np.int64)
    for s in range(SLICES):
        for k in range(J):
            for rt in range(n_rt):
                u = (s * J + k) * n_rt + rt
                off, L = int(table[2 * u]), int(table[2 * u + 1])
                block = entries[off * 64:(off + L) * 64].reshape(L, 64).astype(np.int64)
                for lane in range(64):
                    row = rt * 64 + lane
                    for e in block[:, lane]:
                        jl = e >> SLICE_BITS
                        if jl == Z:
                            continue
                        assert row < out and codes[row, k * Gb + jl] == -1
                        codes[row, k * Gb + jl] = (s << SLICE_BITS) | (e & ((1 << SLICE_BITS) - 1))
    assert (codes >= 0).all()
    return codes.astype(np.uint16).view(np.int16).reshape(out, G, 1)
