"""GPU: the two-pass prefill product aqlm_linear_gemm_dequant (decode W once, then a dense fp16 product).

* outputs meet the GEMM bar against the oracle (relative L2 <= 1e-3, max abs
  <= 1e-2 max|y_ref|): every output on small and ragged problems (several row
  and token tiles, tile counts not a multiple of the XCD count, a single
  k-step), sampled rows at the Llama-2 7B prefill shapes (2048 tokens);
* with dyadic one-hot codebooks and X = identity, Y equals W16 transposed
  exactly (one nonzero product per output);
* the workspace holds the bit-exact decoded weights afterwards; in % 64 != 0
  runs aqlm_linear_gemm (bit-identical) and leaves the workspace alone;
* results are deterministic; bad workspaces are rejected.
"""
import numpy as np
import pytest
import torch

import extreme_weight_quantization_amd as E
from extreme_weight_quantization_amd import synth
from oracle import aqlm_oracle as O

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


def dev(L):
    return tuple(torch.from_numpy(a).cuda() for a in (L.codes, L.codebooks, L.scales, L.x))


def run(L, workspace=None):
    codes, cb, s, x = dev(L)
    y = E.aqlm_linear_gemm_dequant(codes, cb, s, x, workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("out,n_in,batch", [
    (256, 512, 1),      # the tiny layer, one token
    (300, 4160, 130),   # ragged rows and tokens, 65 k-steps
    (128, 256, 256),    # whole tiles
    (200, 64, 70),      # a single k-step
    (1000, 1024, 513),  # 8 row tiles x 3 token tiles (24 tiles, 3 per XCD), ragged
    (129, 128, 257),    # 4 tiles on a grid of 8 (workgroups past the tiles exit)
    (1, 64, 1),         # smallest problem
])
def test_gemm_dequant_small(scheme, out, n_in, batch):
    L = synth.make_layer(scheme, out, n_in, batch=batch, seed=out + batch)
    assert_close(run(L), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), f"{scheme} {out}x{n_in} T{batch}")


@pytest.mark.parametrize("M,B,g", [(1, 8, 4), (4, 8, 16), (2, 16, 32), (3, 5, 8)])
def test_gemm_dequant_generic(M, B, g):
    L = synth.make_layer_mbg(M, B, g, 131, 576, batch=37, seed=M * 16 + B)
    assert_close(run(L), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), f"{M}x{B} g{g}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
def test_gemm_dequant_basis_exact(scheme):
    """X = identity rows: Y equals W16 transposed exactly with dyadic one-hot codebooks."""
    M, B, g, _ = synth.SCHEMES[scheme]
    cb = np.zeros((M, 1 << B, g), np.float16)
    k = np.arange(1 << B)
    for m in range(M):
        cb[m, k, k % 8] = (2.0 ** -(m + 1)) * (((k >> 3) % 32) + 1) / 32
    L = synth.make_layer(scheme, 72, 192, batch=192, seed=3)
    L.codebooks = cb
    L.scales = np.random.default_rng(1).choice([0.5, 1.0, 2.0], size=72).astype(np.float16)
    L.x = np.eye(192, dtype=np.float16)
    np.testing.assert_array_equal(run(L), O.decode_fp16(L.codes, L.codebooks, L.scales).astype(np.float64).T)


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("shape", synth.LLAMA2_7B_SHAPES)
def test_gemm_dequant_prefill_7b(scheme, shape):
    out, n_in = shape
    L = synth.make_layer(scheme, out, n_in, batch=2048, seed=0)
    y = run(L)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(out, 40, replace=False), [0, 127, 128, out - 1]]))
    assert_close(y[:, rows], O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, L.x, rows), f"{scheme} {shape}")


def test_gemm_dequant_workspace_holds_decoded_weights():
    L = synth.make_layer("2x8", 300, 1024, batch=40, seed=9)
    ws = torch.full((E.gemm_dequant_workspace_bytes(2, 8, 8, 300, 1024),), 255, dtype=torch.uint8, device="cuda")
    run(L, ws)
    w16 = ws.view(torch.float16).view(300, 1024).cpu().numpy()
    np.testing.assert_array_equal(w16.view(np.uint16), O.decode_fp16(L.codes, L.codebooks, L.scales).view(np.uint16))


def test_gemm_dequant_unaligned_in_runs_the_fused_product():
    L = synth.make_layer("2x8", 100, 520, batch=5, seed=4)
    codes, cb, s, x = dev(L)
    ws = torch.full((64,), 7, dtype=torch.uint8, device="cuda")
    y = E.aqlm_linear_gemm_dequant(codes, cb, s, x, workspace=ws)
    y_ref = E.aqlm_linear_gemm(codes, cb, s, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert (ws == 7).all()


def test_gemm_dequant_deterministic_and_matches_fused_kernel():
    L = synth.make_layer("1x16", 512, 2048, batch=300, seed=5)
    a, b = run(L), run(L)
    np.testing.assert_array_equal(a, b)
    codes, cb, s, x = dev(L)
    y = E.aqlm_linear_gemm(codes, cb, s, x).cpu().numpy().astype(np.float64)
    assert_close(a, y, "two-pass vs fused")


def test_gemm_dequant_rejects_bad_workspace():
    L = synth.make_layer("2x8", 64, 256, batch=3, seed=0)
    codes, cb, s, x = dev(L)
    need = E.gemm_dequant_workspace_bytes(2, 8, 8, 64, 256)
    with pytest.raises(ValueError):
        E.aqlm_linear_gemm_dequant(codes, cb, s, x, workspace=torch.empty(need - 16, dtype=torch.uint8, device="cuda"))
    big = torch.empty(need + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        E.aqlm_linear_gemm_dequant(codes, cb, s, x, workspace=big[8:])      # not 16-byte aligned
    y0 = E.aqlm_linear_gemm_dequant(codes, cb, s, x[:0])
    assert y0.shape == (0, 64)
