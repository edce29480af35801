"""The slice-list layout reference (tests/lists_layout.py) against its definition (CPU only).

The layout regroups the codes of a 1x16 layer by codebook slice; these tests
pin the reference packer that the GPU tests compare the library with: a
hand-worked example, the round trip back to the codes, and the table's
invariants.
"""
import numpy as np
import pytest

import lists_layout as LL
from extreme_weight_quantization_amd import synth


def codes16(out, n_in, seed):
    return synth.make_layer_mbg(1, 16, 8, out, n_in, seed=seed).codes


def test_hand_worked_example():
    """Two rows, two groups: row 0 = (slice 0, local 5), (slice 3, local 7); row 1 = (3, 1), (3, 2)."""
    c = np.array([[0 << 13 | 5, 3 << 13 | 7], [3 << 13 | 1, 3 << 13 | 2]], np.uint16)
    table, entries = LL.pack(c.view(np.int16).reshape(2, 2, 1), 16)
    pad = 64 << 13          # Z = 64: the 2-group block rounded up to a multiple of 64
    # units u = s (J = 1, one row tile): (off, L)
    want = [(0, 1), (1, 0), (1, 0), (1, 2), (3, 0), (3, 0), (3, 0), (3, 0)]
    assert [(int(table[2 * u]), int(table[2 * u + 1])) for u in range(8)] == want
    assert int(table[16:18].view(np.uint64)[0]) == 3
    e = entries.reshape(3, 64)
    assert e[0, 0] == 5 and e[0, 1] == pad                    # unit 0, step 0
    assert e[1, 0] == (1 << 13 | 7) and e[1, 1] == 1          # unit 3, step 0
    assert e[2, 0] == pad and e[2, 1] == (1 << 13 | 2)        # unit 3, step 1
    assert (e[:, 2:] == pad).all()                            # rows past out are padding


@pytest.mark.parametrize("G,J,Gb,Z", [(1, 1, 1, 64), (64, 1, 64, 64), (1024, 1, 1024, 1024),
                                      (1025, 2, 513, 576), (1376, 2, 688, 704), (3584, 4, 896, 896)])
def test_geometry(G, J, Gb, Z):
    assert LL.geometry(100, 8 * G)[:4] == (G, J, Gb, Z)
    assert (J - 1) * Gb < G        # every block holds at least one group


@pytest.mark.parametrize("out,n_in", [(64, 512), (1, 8), (130, 72), (100, 8800), (65, 8200), (3, 16384)])
def test_round_trip(out, n_in):
    codes = codes16(out, n_in, seed=out + n_in)
    table, entries = LL.pack(codes, n_in)
    np.testing.assert_array_equal(LL.unpack(table, entries, out, n_in), codes)


@pytest.mark.parametrize("out,n_in", [(200, 4096), (64, 8800)])
def test_table_invariants(out, n_in):
    """off is the exclusive prefix of L; L is the longest list of the unit; the total is the sum."""
    codes = codes16(out, n_in, seed=1)
    table, entries = LL.pack(codes, n_in)
    G, J, Gb, Z, n_rt = LL.geometry(out, n_in)
    n = 8 * J * n_rt
    off, L = table[0:2 * n:2].astype(np.int64), table[1:2 * n:2].astype(np.int64)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(L)[:-1]]))
    assert int(table[2 * n:2 * n + 2].view(np.uint64)[0]) == L.sum() == entries.size // 64
    c = codes.reshape(out, G).view(np.uint16).astype(np.int64)
    for s in range(8):
        for k in range(J):
            for rt in range(n_rt):
                blk = c[rt * 64:rt * 64 + 64, k * Gb:(k + 1) * Gb]
                assert L[(s * J + k) * n_rt + rt] == ((blk >> 13) == s).sum(1).max()
    # every code appears once: the listed entries number out * G
    assert (entries >> 13 != Z).sum() == out * G


def test_uniform_codes_pad_by_a_quarter_or_less():
    """Uniform 1x16 codes at the 7B width: padding to the longest of 64 lists costs < 35 % of the entries."""
    codes = codes16(256, 4096, seed=2)
    _, entries = LL.pack(codes, 4096)
    assert entries.size / codes.size < 1.35
