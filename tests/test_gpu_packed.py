"""GPU parity of the bit-packed code path, through the C ABI, against the CPU oracle.

* aqlm_pack_codes writes the same word stream as the oracle's pack_codes, bit
  for bit (junk in the unused high bits of the stored codes is dropped);
* aqlm_linear_decode_packed is bit-exact against the oracle's decode of the
  packed stream;
* aqlm_linear_gemv_packed / aqlm_linear_gemm_packed meet the GEMV/GEMM bar
  (relative L2 <= 1e-3, max abs <= 1e-2 max|y_ref|) over every output;
* on full 4096x4096 and 4096x11008 layers of (1,12,4), (3,5,8) and (2,12,8),
  every output, and the stream is 8 * bytes / weights = M B / g bits per weight.
The oracle's packed stream is what the kernels read in the product tests, so
the packing kernel and the products are checked independently.
"""
import numpy as np
import pytest
import torch

import extreme_weight_quantization_amd as E
from extreme_weight_quantization_amd import synth
from oracle import aqlm_oracle as O
from parity_util import assert_close_all

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X")
    E.load_library()
    torch.cuda.init()


def junk_high_bits(codes, B, seed):
    rng = np.random.default_rng(seed)
    bits = 8 if codes.dtype == np.uint8 else 16
    if B == bits:
        return codes.copy()
    u = codes.view(np.uint8 if bits == 8 else np.uint16).astype(np.int64)
    out = (u | (rng.integers(0, 1 << (bits - B), size=u.shape) << B)).astype(np.uint8 if bits == 8 else np.uint16)
    return out if bits == 8 else out.view(np.int16)


def words_dev(words):
    return torch.from_numpy(words.view(np.int32).copy()).cuda()


def dev_layer(L, words):
    return (words_dev(words), torch.from_numpy(L.codebooks).cuda(), torch.from_numpy(L.scales).cuda(),
            torch.from_numpy(L.x).cuda())


SCHEMES = [(1, 12, 4), (3, 5, 8), (2, 12, 8), (1, 3, 2), (2, 7, 16), (1, 16, 8), (2, 8, 8), (5, 9, 32), (1, 1, 1)]


@pytest.mark.parametrize("M,B,g", SCHEMES)
def test_pack_codes_bit_exact(M, B, g):
    L = synth.make_layer_mbg(M, B, g, 37, 13 * g, seed=M + B)
    codes = junk_high_bits(L.codes, B, seed=3)
    packed = E.aqlm_pack_codes(torch.from_numpy(codes).cuda(), B)
    torch.cuda.synchronize()
    want = O.pack_codes(codes, B)
    got = packed.cpu().numpy().view(np.uint32)
    assert got.size == max(want.size, 1)
    np.testing.assert_array_equal(got[:want.size], want)


@pytest.mark.parametrize("M,B,g", SCHEMES)
def test_decode_packed_bit_exact(M, B, g):
    out, n_in = 53, 11 * g * (8 if g < 8 else 1)
    L = synth.make_layer_mbg(M, B, g, out, n_in, seed=2 * M + B)
    words = O.pack_codes(L.codes, B)
    p, cb, s, _ = dev_layer(L, words)
    w = E.aqlm_linear_decode_packed(p, cb, s, n_in)
    torch.cuda.synchronize()
    want = O.decode_fp32_packed(words, L.codebooks, L.scales, M, B, g, out, n_in).astype(np.float16)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M,B,g", SCHEMES)
@pytest.mark.parametrize("batch", [1, 5, 16])
def test_gemv_packed(M, B, g, batch):
    out, n_in = 70, 9 * g * 8
    L = synth.make_layer_mbg(M, B, g, out, n_in, batch=batch, seed=M * B + batch)
    words = O.pack_codes(L.codes, B)
    y = E.aqlm_linear_gemv_packed(*dev_layer(L, words)).cpu().numpy()
    want = O.linear_ref_f64(O.packed_to_stored(words, M, B, g, out, n_in), L.codebooks, L.scales, L.x)
    assert_close_all(y, want, f"gemv {M}x{B}g{g} T{batch}")


@pytest.mark.parametrize("M,B,g", SCHEMES)
@pytest.mark.parametrize("out,n_grp,batch", [(200, 37, 130), (64, 8, 3)])
def test_gemm_packed(M, B, g, out, n_grp, batch):
    n_in = n_grp * g
    L = synth.make_layer_mbg(M, B, g, out, n_in, batch=batch, seed=M + B + batch)
    words = O.pack_codes(L.codes, B)
    y = E.aqlm_linear_gemm_packed(*dev_layer(L, words)).cpu().numpy()
    want = O.linear_ref_f64(O.packed_to_stored(words, M, B, g, out, n_in), L.codebooks, L.scales, L.x)
    assert_close_all(y, want, f"gemm {M}x{B}g{g} {out}x{n_in} T{batch}")


@pytest.mark.parametrize("M,B,g", [(1, 12, 4), (3, 5, 8), (2, 12, 8)])
@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 11008)])
def test_packed_full_size(M, B, g, shape):
    """Full layers: the packing kernel against the oracle, decode bit-exact, GEMV at batch 1 and 16 and
    a 2048-token GEMM (4096x4096 only) over every output; the stream costs exactly M B / g bits per weight."""
    out, n_in = shape
    L = synth.make_layer_mbg(M, B, g, out, n_in, batch=16, seed=M * 31 + B)
    words = O.pack_codes(L.codes, B)
    assert 8 * words.nbytes == M * B * out * n_in // g
    packed = E.aqlm_pack_codes(torch.from_numpy(L.codes).cuda(), B)
    p, cb, s, x = dev_layer(L, words)
    w = E.aqlm_linear_decode_packed(p, cb, s, n_in)
    y16 = E.aqlm_linear_gemv_packed(p, cb, s, x)
    y1 = E.aqlm_linear_gemv_packed(p, cb, s, x[:1].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), words)
    stored = O.packed_to_stored(words, M, B, g, out, n_in)
    chunks = [np.arange(r, min(r + 1024, out)) for r in range(0, out, 1024)]
    w_ref = np.concatenate([O.decode_fp16(stored, L.codebooks, L.scales, rows=c) for c in chunks])
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), w_ref.view(np.uint16))
    y_ref = np.concatenate([O.linear_ref_rows_f64(stored, L.codebooks, L.scales, L.x, c) for c in chunks], axis=1)
    assert_close_all(y16.cpu().numpy(), y_ref, "gemv b16")
    assert_close_all(y1.cpu().numpy(), y_ref[:1], "gemv b1")
    if shape == (4096, 4096):
        xs_h = synth.make_activations(n_in, 2048, seed=1)
        yg = E.aqlm_linear_gemm_packed(p, cb, s, torch.from_numpy(xs_h).cuda())
        yg_ref = np.concatenate([O.linear_ref_rows_f64(stored, L.codebooks, L.scales, xs_h, c) for c in chunks],
                                axis=1)
        assert_close_all(yg.cpu().numpy(), yg_ref, "gemm 2048")


def test_packed_errors():
    L = synth.make_layer_mbg(1, 12, 4, 64, 512, batch=1, seed=1)
    words = O.pack_codes(L.codes, 12)
    p, cb, s, x = dev_layer(L, words)
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv_packed(p[:10].contiguous(), cb, s, x)          # stream too short for the layer
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv_packed(p.to(torch.int64), cb, s, x)
    with pytest.raises(ValueError):
        E.aqlm_pack_codes(torch.from_numpy(L.codes).cuda(), 8)            # int16 codes with B = 8
    torch.cuda.synchronize()
