"""The allocation-free slice-list product (aqlm_linear_gemv_lists_noalloc), through the C ABI.

Its partial sums live in the library's static device array instead of a caller
workspace.  Checked against the workspace entry point it shares its kernels with
(bit for bit) and against the oracle, on two calls in a row, the second with a
smaller layer (stale scratch from the first must not leak into it), then the first
shape again; an oversized layer is refused with AQLM_ERR_SCRATCH.
"""
import ctypes

import numpy as np
import pytest
import torch

import extreme_weight_quantization_amd as E
from extreme_weight_quantization_amd import binding, synth
from oracle import aqlm_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X")
    E.load_library()


def _noalloc_raw(lists, cb, s, x, y, out, n_in, batch=1):
    lib = E.load_library()
    return int(lib.aqlm_linear_gemv_lists_noalloc(
        ctypes.c_void_p(lists.table.data_ptr()), ctypes.c_void_p(lists.entries.data_ptr()), lists.entries.numel(),
        ctypes.c_void_p(cb.data_ptr()), ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(x.data_ptr()),
        ctypes.c_void_p(y.data_ptr()), 1, 16, 8, out, n_in, batch,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))


def _case(out, n_in, seed):
    L = synth.make_layer("1x16", out, n_in, batch=1, seed=seed)
    codes = torch.from_numpy(L.codes).cuda()
    cb = torch.from_numpy(L.codebooks).cuda()
    s = torch.from_numpy(L.scales).cuda()
    x = torch.from_numpy(L.x).cuda()
    lists = E.aqlm_lists_pack(codes)
    return L, lists, cb, s, x


@pytest.mark.parametrize("shapes", [((4096, 4096), (300, 1032)), ((11008, 4096), (4096, 11008))])
def test_noalloc_matches_workspace_entry_point_and_oracle(shapes):
    results = []
    for i, (out, n_in) in enumerate(list(shapes) + [shapes[0]]):
        L, lists, cb, s, x = _case(out, n_in, seed=10 + i % 2)
        y = torch.full((1, out), float("nan"), dtype=torch.float16, device="cuda")
        assert _noalloc_raw(lists, cb, s, x, y, out, n_in) == binding.AQLM_OK
        want = E.aqlm_linear_gemv_lists(lists, cb, s, x)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.cpu().numpy().view(np.uint16)), (out, n_in)
        y_ref = O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
        rel, mx, ref_max = O.parity_errors(got.astype(np.float64), y_ref)
        assert rel <= 1e-3 and mx <= 1e-2 * ref_max, (out, n_in, rel, mx)
        results.append(got)
    assert np.array_equal(results[0].view(np.uint16), results[2].view(np.uint16))


def test_noalloc_refuses_layers_beyond_its_scratch():
    out, n_in = 200000, 64     # 8 slices x 3125 row tiles x 64 rows x 4 B = 6.4 MB > 4 MiB
    assert E.lists_workspace_bytes(out, n_in) > binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, n_in), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, 16), dtype=torch.float16, device="cuda")
    lib = E.load_library()
    st = lib.aqlm_linear_gemv_lists_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), 0,
                                            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                                            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                            1, 16, 8, out, n_in, 1, None)
    assert st == binding.AQLM_ERR_SCRATCH
    assert "scratch" in binding.status_str(st)
