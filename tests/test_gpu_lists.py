"""GPU: the 1x16 slice-list path (aqlm_lists_plan / aqlm_lists_fill / aqlm_linear_gemv_lists).

* the table and entries the library writes equal, byte for byte, the layout
  reference in tests/lists_layout.py (integer work: bit-exact);
* the product meets the GEMV bar against the oracle (relative L2 <= 1e-3,
  max abs <= 1e-2 max|y_ref|): every output on small and ragged layers,
  sampled rows at the Llama-2 7B/70B shapes in the launch configuration the
  benchmark times;
* single-term sums are exact (one-hot x on dyadic codebooks), results are
  deterministic, and undersized buffers read nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import extreme_weight_quantization_amd as E
import lists_layout as LL
from extreme_weight_quantization_amd import synth
from oracle import aqlm_oracle as O
from parity_util import assert_close_all, ref_full

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS_FRAC = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X")
    E.load_library()
    torch.cuda.init()


def assert_close(y, y_ref, what=""):
    rel, mx, ref_max = O.parity_errors(y, y_ref)
    assert np.isfinite(rel), what
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC * ref_max, f"{what}: max abs {mx:.3e} > 1e-2 * {ref_max:.3e}"


def sample_rows(out, n=96, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(out, size=min(n, out), replace=False).tolist())
    rows |= {0, out - 1, min(63, out - 1), min(64, out - 1)}
    return np.array(sorted(rows), dtype=np.int64)


def run(layer, lists=None):
    codes = torch.from_numpy(layer.codes).cuda()
    cb = torch.from_numpy(layer.codebooks).cuda()
    s = torch.from_numpy(layer.scales).cuda()
    x = torch.from_numpy(layer.x).cuda()
    if lists is None:
        lists = E.aqlm_lists_pack(codes)
    y = E.aqlm_linear_gemv_lists(lists, cb, s, x)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), lists


SMALL = [(256, 512), (1, 8), (130, 72), (100, 8800), (65, 8200), (64, 512), (3, 16384), (700, 136), (4096 + 8, 256)]


@pytest.mark.parametrize("out,n_in", SMALL)
def test_pack_bit_exact(out, n_in):
    L = synth.make_layer("1x16", out, n_in, seed=out)
    lists = E.aqlm_lists_pack(torch.from_numpy(L.codes).cuda())
    table, entries = LL.pack(L.codes, n_in)
    np.testing.assert_array_equal(lists.table.cpu().numpy().view(np.uint32), table)
    np.testing.assert_array_equal(lists.entries.cpu().numpy().view(np.uint32), entries)


@pytest.mark.parametrize("out,n_in", SMALL)
def test_gemv_lists_small(out, n_in):
    L = synth.make_layer("1x16", out, n_in, seed=out + 1)
    y, _ = run(L)
    assert_close(y, O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), f"{out}x{n_in}")


def test_gemv_lists_basis_vectors_exact():
    """Dyadic one-hot codewords: x = e_k makes y the column k of W16, exactly (one nonzero product per row)."""
    cb = np.zeros((1, 65536, 8), np.float16)
    k = np.arange(65536)
    cb[0, k, k % 8] = (((k >> 3) % 32) + 1) / 64
    L = synth.make_layer("1x16", 200, 9000, seed=3)       # two blocks of groups, a ragged row tile
    L.codebooks = cb
    L.scales = np.random.default_rng(0).choice([0.5, 1.0, 1.5, 2.0], size=200).astype(np.float16)
    w16 = O.decode_fp16(L.codes, L.codebooks, L.scales).astype(np.float64)
    lists = None
    for col in (0, 7, 8, 4495, 4496, 4503, 8999):
        L.x = np.zeros((1, 9000), np.float16)
        L.x[0, col] = 1
        y, lists = run(L, lists)
        np.testing.assert_array_equal(y[0], w16[:, col])


def test_gemv_lists_long_parts_full():
    """520 x 262144: 32 blocks of 1024 groups, one workgroup per (slice, block), 9 row tiles (the last
    ragged), undivided parts of ~160 steps: the two-ring path, every output against the oracle."""
    L = synth.make_layer("1x16", 520, 262144, seed=13)
    y, _ = run(L)
    assert_close(y, O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), "520x262144")


@pytest.mark.parametrize("shape", synth.LLAMA2_7B_SHAPES)
def test_gemv_lists_7b(shape):
    out, n_in = shape
    L = synth.make_layer("1x16", out, n_in, batch=1, seed=0)
    y, _ = run(L)
    assert_close_all(y, ref_full(L), str(shape))
    codes = torch.from_numpy(L.codes).cuda()
    y_plain = E.aqlm_linear_gemv(codes, torch.from_numpy(L.codebooks).cuda(), torch.from_numpy(L.scales).cuda(),
                                 torch.from_numpy(L.x).cuda()).cpu().numpy().astype(np.float64)
    assert_close(y, y_plain, f"{shape} vs aqlm_linear_gemv")


@pytest.mark.parametrize("shape", synth.LLAMA2_70B_SHAPES)
def test_gemv_lists_70b(shape):
    out, n_in = shape
    L = synth.make_layer("1x16", out, n_in, batch=1, seed=0)
    y, _ = run(L)
    assert_close_all(y, ref_full(L), str(shape))


def test_pack_70b_down_entries_sampled():
    """8192 x 28672 (four blocks of 896 groups): sampled units of the library's table and entries
    equal the reference's (the reference packs the same codes in full on the CPU)."""
    L = synth.make_layer("1x16", 8192, 28672, seed=0)
    lists = E.aqlm_lists_pack(torch.from_numpy(L.codes).cuda())
    table, entries = LL.pack(L.codes, 28672)
    got_t = lists.table.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got_t, table)
    got_e = lists.entries.view(torch.int32)
    rng = np.random.default_rng(1)
    n_units = (table.size - 2) // 2
    for u in rng.choice(n_units, 24, replace=False):
        off, n = int(table[2 * u]), int(table[2 * u + 1])
        np.testing.assert_array_equal(got_e[off * 64:(off + n) * 64].cpu().numpy().view(np.uint32),
                                      entries[off * 64:(off + n) * 64])


def test_gemv_lists_deterministic_and_reusable():
    L = synth.make_layer("1x16", 4096, 4096, seed=5)
    y1, lists = run(L)
    y2, _ = run(L, lists)
    np.testing.assert_array_equal(y1, y2)


def test_gemv_lists_given_output_workspace_and_stream():
    L = synth.make_layer("1x16", 300, 1024, seed=6)
    codes = torch.from_numpy(L.codes).cuda()
    cb, s, x = (torch.from_numpy(a).cuda() for a in (L.codebooks, L.scales, L.x))
    lists = E.aqlm_lists_pack(codes)
    y = torch.full((1, 300), float("nan"), dtype=torch.float16, device="cuda")
    ws = torch.full((E.lists_workspace_bytes(300, 1024),), 255, dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        E.aqlm_linear_gemv_lists(lists, cb, s, x, y=y, workspace=ws)
    st.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x))


def test_gemv_lists_undersized_entries_read_nothing():
    """entries_bytes = 0: no unit fits, none is read, every partial sum is 0 and y is +0."""
    L = synth.make_layer("1x16", 128, 512, seed=7)
    codes = torch.from_numpy(L.codes).cuda()
    cb, s, x = (torch.from_numpy(a).cuda() for a in (L.codebooks, L.scales, L.x))
    lists = E.aqlm_lists_pack(codes)
    y = torch.full((1, 128), float("nan"), dtype=torch.float16, device="cuda")
    ws = torch.empty(E.lists_workspace_bytes(128, 512), dtype=torch.uint8, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = E.load_library().aqlm_linear_gemv_lists(
        p(lists.table), p(lists.entries), 0, p(cb), p(s), p(x), p(y), p(ws), ws.numel(), 1, 16, 8, 128, 512, 1,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert (y.view(torch.int16) == 0).all()


def test_gemv_lists_empty_batch_and_layer():
    L = synth.make_layer("1x16", 64, 512, seed=8)
    codes = torch.from_numpy(L.codes).cuda()
    cb, s = torch.from_numpy(L.codebooks).cuda(), torch.from_numpy(L.scales).cuda()
    lists = E.aqlm_lists_pack(codes)
    y = E.aqlm_linear_gemv_lists(lists, cb, s, torch.zeros((0, 512), dtype=torch.float16, device="cuda"))
    assert y.shape == (0, 64)
    z = E.aqlm_lists_pack(torch.zeros((0, 64, 1), dtype=torch.int16, device="cuda"))
    assert z.steps == 0 and z.table.numel() == 8


@pytest.mark.parametrize("outs,n_in", [((4096, 4096, 4096), 4096), ((11008, 11008), 4096), ((300, 0, 65, 1), 9000),
                                       ((1024, 8192), 8192)])
def test_gemv_lists_fused_matches_separate_and_oracle(outs, n_in):
    """One launch for layers that share x: bit-identical to separate calls; sampled rows against the oracle."""
    x = synth.make_activations(n_in, 1, seed=11)
    xd = torch.from_numpy(x).cuda()
    layers, devs, hosts = [], [], []
    for li, out in enumerate(outs):
        L = synth.make_layer("1x16", out, n_in, seed=20 + li)
        cb, s = torch.from_numpy(L.codebooks).cuda(), torch.from_numpy(L.scales).cuda()
        lists = E.aqlm_lists_pack(torch.from_numpy(L.codes).cuda())
        layers.append((lists, cb, s))
        hosts.append(L)
    ys = E.aqlm_linear_gemv_lists_fused(layers, xd)
    torch.cuda.synchronize()
    for (lists, cb, s), y, L in zip(layers, ys, hosts):
        if L.out_features == 0:
            assert y.shape == (1, 0)
            continue
        y_sep = E.aqlm_linear_gemv_lists(lists, cb, s, xd)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_sep.view(torch.int16))
        rows = sample_rows(L.out_features, 48)
        got = y.cpu().numpy().astype(np.float64)[:, rows]
        assert_close(got, O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, x, rows), f"fused {outs}")
