"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests touches the GPU.  Each pin is chosen so that a plausible
slip in the oracle (a dropped codebook, codes read in the wrong order, the
scale applied per column, int16 codes read as signed, a sum started from +0,
a transposed product) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import aqlm_oracle as O
from extreme_weight_quantization_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(vals):
    return np.array([(-0.0 if v == "-0" else v) for v in vals], dtype=np.float16)


# --------------------------------------------------------------------------
# Decode


def test_worked_example_2x8():
    """Hand-worked decode and product from the MCQ section's Figure 2."""
    ex = _load("worked_2x8.json")
    M, B, g = ex["M"], ex["B"], ex["g"]
    cb = np.zeros((M, 1 << B, g), dtype=np.float16)
    for key, vals in ex["codebook_entries"].items():
        m, k = (int(v) for v in key.split(":"))
        cb[m, k] = _f16(vals)
    codes = np.array(ex["codes"], dtype=np.uint8)
    scales = np.array(ex["scales"], dtype=np.float16)
    x = np.array(ex["x"], dtype=np.float16)
    want = np.array([_f16(r) for r in ex["W"]]).astype(np.float32)
    w = O.decode_fp32(codes, cb, scales)
    assert w.dtype == np.float32
    np.testing.assert_array_equal(w, want)
    assert np.array_equal(np.signbit(w), np.signbit(want)), "signed zeros differ"
    w16 = O.decode_fp16(codes, cb, scales)
    assert np.array_equal(w16.view(np.uint16), want.astype(np.float16).view(np.uint16))
    y = O.linear_ref_f64(codes, cb, scales, x)
    np.testing.assert_array_equal(y, np.array(ex["y"], dtype=np.float64))


def test_vectorised_matches_loops_config_tiny_2x8():
    """256x512 2x8 layer, seed 0: gather decode equals the explicit-loop decode bit for bit."""
    L = synth.make_layer("2x8", 256, 512, batch=1, seed=0)
    assert L.codes.shape == (256, 64, 2) and L.codes.dtype == np.uint8
    a = O.decode_fp32(L.codes[:24], L.codebooks, L.scales[:24])
    b = O.decode_loop(L.codes[:24], L.codebooks, L.scales[:24])
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_vectorised_matches_loops_1x16():
    L = synth.make_layer("1x16", 8, 64, seed=3)
    a = O.decode_fp32(L.codes, L.codebooks, L.scales)
    b = O.decode_loop(L.codes, L.codebooks, L.scales)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


GENERIC = [(1, 8, 4), (4, 8, 16), (8, 8, 32), (3, 5, 8), (1, 12, 4), (2, 16, 32)]


def _junk_high_bits(codes, B, seed):
    """Set the unused high bits of every stored code at random (the index is the low B bits)."""
    rng = np.random.default_rng(seed)
    bits = 8 if codes.dtype == np.uint8 else 16
    if B == bits:
        return codes.copy()
    u = codes.view(np.uint8 if bits == 8 else np.uint16).astype(np.int64)
    junk = rng.integers(0, 1 << (bits - B), size=u.shape) << B
    out = (u | junk).astype(np.uint8 if bits == 8 else np.uint16)
    return out if bits == 8 else out.view(np.int16)


@pytest.mark.parametrize("M,B,g", GENERIC + [(1, 12, 1), (3, 5, 2)])
def test_vectorised_matches_loops_generic(M, B, g):
    """Gather decode = explicit loops, bit for bit, for budget-equivalent and odd schemes."""
    L = synth.make_layer_mbg(M, B, g, 6, 4 * g * 4, seed=M * 100 + B)
    codes = _junk_high_bits(L.codes, B, seed=7)
    a = O.decode_fp32(codes, L.codebooks, L.scales)
    b = O.decode_loop(codes, L.codebooks, L.scales)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M,B,g", GENERIC)
def test_index_layout_generic_spelled_codes(M, B, g):
    """Codebook m spells its index k in entries 2m (k >> 8) and 2m+1 (k & 255), zero elsewhere.

    With scale 1 the decoded group holds every code of the group exactly, so
    decoding recovers the code array: this pins the [out][G][M] layout, which
    codebook each of the M codes indexes, the column order j*g + t for any g,
    and the reading that only the low B bits of a stored code count (the
    codes carry random junk in their unused high bits).
    """
    K = 1 << B
    k = np.arange(K)
    cb = np.zeros((M, K, g), np.float16)
    for m in range(M):
        cb[m, :, 2 * m] = k >> 8
        cb[m, :, 2 * m + 1] = k & 255
    L = synth.make_layer_mbg(M, B, g, 5, 3 * g, seed=11)
    codes = _junk_high_bits(L.codes, B, seed=12)
    w = O.decode_fp32(codes, cb, np.ones(5, np.float16)).reshape(5, 3, g)
    got = np.stack([256 * w[:, :, 2 * m] + w[:, :, 2 * m + 1] for m in range(M)], axis=-1).astype(np.int64)
    want = O.codes_to_index(L.codes)      # the drawn codes, all < 2^B
    np.testing.assert_array_equal(got, want)
    assert np.all(w[:, :, 2 * M:] == 0)


@pytest.mark.parametrize("M,B,g", GENERIC)
def test_all_ones_generic_closed_form(M, B, g):
    """All-ones codebooks: W[i][k] = M * s_i and y_i = M * s_i * sum(x) for any scheme."""
    L = synth.make_layer_mbg(M, B, g, 7, 2 * g * 3, batch=2, seed=5)
    cb = np.ones((M, 1 << B, g), np.float16)
    w = O.decode_fp32(L.codes, cb, L.scales)
    np.testing.assert_array_equal(w, np.repeat((M * L.scales.astype(np.float32))[:, None], w.shape[1], 1))
    y = O.linear_ref_f64(L.codes, cb, L.scales, L.x)
    want = M * L.scales.astype(np.float64)[None, :] * L.x.astype(np.float64).sum(1)[:, None]
    np.testing.assert_allclose(y, want, rtol=1e-12)


def test_budget_equivalent_pairs_code_bits():
    """"Key AQLM quantization parameters": at B = 8 the pairs (1,4), (2,8), ..., (8,32) cost 2 code bits."""
    for M, g in ((1, 4), (2, 8), (4, 16), (8, 32)):
        assert O.bits_per_weight_terms(M, 8, g, 28672, 8192)["codes"] == 2.0


def test_index_layout_2x8_bit_codebooks():
    """C0[k][t] = bit t of k, C1[k][t] = 2 * bit t of k: each decoded group spells out its two codes.

    Pins the [out][G][M] code layout, the codebook order and the column order
    j*g + t: the codes are recovered exactly from the decoded weights.
    """
    g, K = 8, 256
    k = np.arange(K)[:, None]
    t = np.arange(g)[None, :]
    bits = ((k >> t) & 1).astype(np.float16)
    cb = np.stack([bits, 2 * bits]).astype(np.float16)
    rng = np.random.default_rng(7)
    out, G = 5, 6
    codes = rng.integers(0, 256, size=(out, G, 2), dtype=np.uint8)
    w = O.decode_fp32(codes, cb, np.ones(out, np.float16)).reshape(out, G, g).astype(np.int64)
    a = ((w % 2) << t[None]).sum(-1)
    b = ((w // 2) << t[None]).sum(-1)
    assert np.array_equal(a, codes[:, :, 0]) and np.array_equal(b, codes[:, :, 1])


def test_index_reading_int16_codes():
    """1x16: C[k][t] = 2-bit digit t of k.  Decoding recovers the int16 code as an unsigned index."""
    g = 8
    k = np.arange(1 << 16)[:, None]
    t = np.arange(g)[None, :]
    cb = ((k >> (2 * t)) & 3).astype(np.float16)[None]
    codes = np.array([[[0], [1], [-1], [-32768], [32767], [12345], [-2]]], dtype=np.int16)
    w = O.decode_fp32(codes, cb, np.ones(1, np.float16)).reshape(1, 7, g).astype(np.int64)
    idx = (w << (2 * t[None])).sum(-1)
    assert idx.tolist() == [[0, 1, 65535, 32768, 32767, 12345, 65534]]
    np.testing.assert_array_equal(O.codes_to_index(codes)[0, :, 0], [0, 1, 65535, 32768, 32767, 12345, 65534])


def test_one_hot_dyadic_brute_force():
    """Dyadic one-hot codebooks: codeword k of codebook m is 2^-(m+1) * ((k>>3)+1)/32 * e_(k mod 8).

    With scales in {0.5, 1, 1.5, 2} every sum and product is exact, so a dense
    float64 product with the identity returns each weight, which must equal
    the value worked out entry by entry from the construction.
    """
    M, K, g = 2, 256, 8
    cb = np.zeros((M, K, g), dtype=np.float16)
    for m in range(M):
        for k in range(K):
            cb[m, k, k % 8] = 2.0 ** -(m + 1) * ((k >> 3) + 1) / 32
    rng = np.random.default_rng(11)
    out, n_in = 4, 16
    codes = rng.integers(0, 256, size=(out, n_in // g, M), dtype=np.uint8)
    scales = rng.choice([0.5, 1.0, 1.5, 2.0], size=out).astype(np.float16)
    Y = O.linear_ref_f64(codes, cb, scales, np.eye(n_in, dtype=np.float16))  # [in][out] = W^T
    for i in range(out):
        for j in range(n_in // g):
            for t in range(g):
                want = 0.0
                for m in range(M):
                    b = int(codes[i, j, m])
                    if b % 8 == t:
                        want += 2.0 ** -(m + 1) * ((b >> 3) + 1) / 32
                want *= float(scales[i])
                assert Y[j * g + t, i] == want


def test_all_ones_codebooks_closed_form():
    """All-ones codebooks: every weight is M*s_i, so y_i = M*s_i*sum(x)."""
    for scheme in ("2x8", "1x16"):
        L = synth.make_layer(scheme, 16, 64, batch=3, seed=1)
        cb = np.ones_like(L.codebooks)
        w = O.decode_fp32(L.codes, cb, L.scales)
        np.testing.assert_array_equal(w, np.repeat((L.M * L.scales.astype(np.float32))[:, None], 64, 1))
        y = O.linear_ref_f64(L.codes, cb, L.scales, L.x)
        want = L.M * L.scales.astype(np.float64)[None, :] * L.x.astype(np.float64).sum(1)[:, None]
        np.testing.assert_allclose(y, want, rtol=1e-14, atol=0)


def test_zero_second_codebook_reduces_to_embedding():
    """2x8 with C1 = 0 equals the single-codebook lookup (torch embedding) times the scale."""
    L = synth.make_layer("2x8", 32, 128, seed=2)
    cb = L.codebooks.copy()
    cb[1] = 0
    w = O.decode_fp32(L.codes, cb, L.scales)
    emb = torch.nn.functional.embedding(torch.from_numpy(L.codes[:, :, 0].astype(np.int64)),
                                        torch.from_numpy(cb[0].astype(np.float64)))
    want = (emb * torch.from_numpy(L.scales.astype(np.float64))[:, None, None]).reshape(32, 128)
    np.testing.assert_array_equal(w.astype(np.float64), want.numpy())


def test_1x16_equals_embedding_lookup():
    L = synth.make_layer("1x16", 32, 128, seed=4)
    w = O.decode_fp32(L.codes, L.codebooks, L.scales)
    idx = torch.from_numpy(L.codes[:, :, 0].view(np.uint16).astype(np.int64))
    emb = torch.nn.functional.embedding(idx, torch.from_numpy(L.codebooks[0].astype(np.float64)))
    want = (emb * torch.from_numpy(L.scales.astype(np.float64))[:, None, None]).reshape(32, 128)
    # fp16 x fp16 products are exact in fp32, so the fp64 product equals the fp32 one
    np.testing.assert_array_equal(w.astype(np.float64), want.numpy())


def test_basis_vector_selects_column():
    L = synth.make_layer("2x8", 64, 256, seed=5)
    w = O.decode_fp32(L.codes, L.codebooks, L.scales)
    for k in (0, 7, 8, 100, 255):
        x = np.zeros((1, 256), np.float16)
        x[0, k] = 1
        y = O.linear_ref_f64(L.codes, L.codebooks, L.scales, x)
        np.testing.assert_array_equal(y[0], w[:, k].astype(np.float64))


def test_linearity_in_x_and_scale():
    L = synth.make_layer("2x8", 48, 256, batch=2, seed=6)
    y = O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
    x2 = (L.x.astype(np.float32) * 2).astype(np.float16)  # exact
    y2 = O.linear_ref_f64(L.codes, L.codebooks, L.scales, x2)
    np.testing.assert_array_equal(y2, 2 * y)
    w = O.decode_fp32(L.codes, L.codebooks, L.scales)
    w2 = O.decode_fp32(L.codes, L.codebooks, (L.scales.astype(np.float32) * 4).astype(np.float16))
    np.testing.assert_array_equal(w2, 4 * w)
    # additivity over a sum of inputs, up to float64 rounding
    xa = synth.make_activations(256, 1, seed=1).astype(np.float64)
    xb = synth.make_activations(256, 1, seed=2).astype(np.float64)
    wa = w.astype(np.float64)
    np.testing.assert_allclose(wa @ (xa + xb).T, wa @ xa.T + wa @ xb.T, rtol=1e-12, atol=1e-12)


def test_codebook_permutation_invariance():
    """Permuting codebook entries together with the matching code remap leaves W unchanged."""
    L = synth.make_layer("2x8", 32, 128, seed=8)
    rng = np.random.default_rng(0)
    perms = [rng.permutation(256) for _ in range(2)]
    cb = np.stack([L.codebooks[m][perms[m]] for m in range(2)])
    inv = [np.argsort(p) for p in perms]
    codes = np.stack([inv[m][L.codes[:, :, m]] for m in range(2)], axis=-1).astype(np.uint8)
    a = O.decode_fp32(L.codes, L.codebooks, L.scales)
    b = O.decode_fp32(codes, cb, L.scales)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_codebook_order_matters_only_through_rounding():
    """Swapping the two codebooks (and codes) gives the same fp32 weights: fp32 addition is commutative."""
    L = synth.make_layer("2x8", 16, 64, seed=9)
    a = O.decode_fp32(L.codes, L.codebooks, L.scales)
    b = O.decode_fp32(L.codes[:, :, ::-1].copy(), L.codebooks[::-1].copy(), L.scales)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_signed_zero_and_rne_subnormal_rounding():
    """fp32 sum starts from codebook 0 (keeps -0), and fp16 rounding is nearest-even with subnormals kept."""
    cb = np.zeros((2, 256, 8), np.float16)
    cb[0, 1] = -0.0
    cb[1, 1] = -0.0
    cb[0, 2] = np.float16(2.0 ** -24)      # smallest fp16 subnormal
    cb[1, 2] = np.float16(2.0 ** -24)
    codes = np.array([[[1, 1], [2, 2], [1, 0]]], np.uint8)
    w32 = O.decode_fp32(codes, cb, np.array([1.25], np.float16))
    assert np.all(np.signbit(w32[0, :8])) and np.all(w32[0, :8] == 0)   # (-0)+(-0) = -0
    assert not np.any(np.signbit(w32[0, 16:]))                          # (-0)+(+0) = +0
    # 2*2^-24*1.25 = 2.5 * 2^-24 -> ties to even -> 2 * 2^-24
    w16 = O.decode_fp16(codes, cb, np.array([1.25], np.float16))
    assert np.all(w16[0, 8:16] == np.float16(2.0 ** -23))
    w16b = O.decode_fp16(codes, cb, np.array([1.5], np.float16))   # 3 * 2^-24, exact
    assert np.all(w16b[0, 8:16].view(np.uint16) == 3)


# --------------------------------------------------------------------------
# Matrix product


def test_product_against_fsum():
    L = synth.make_layer("1x16", 64, 512, batch=2, seed=10)
    y = O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
    w = O.decode_fp32(L.codes, L.codebooks, L.scales).astype(np.float64)
    x = L.x.astype(np.float64)
    for b in range(2):
        for i in (0, 17, 63):
            exact = math.fsum(w[i] * x[b])
            assert abs(y[b, i] - exact) <= 1e-12 * max(1.0, math.fsum(abs(w[i] * x[b])))


def test_rows_subset_matches_full():
    L = synth.make_layer("2x8", 40, 128, batch=3, seed=12)
    rows = [0, 5, 39, 17]
    full = O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
    sub = O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, L.x, rows)
    np.testing.assert_array_equal(sub, full[:, rows])


def test_validation_errors():
    L = synth.make_layer("2x8", 8, 64)
    with pytest.raises(ValueError):
        O.decode_fp32(L.codes.astype(np.int16), L.codebooks, L.scales)
    with pytest.raises(ValueError):
        O.decode_fp32(L.codes, L.codebooks.astype(np.float32), L.scales)
    with pytest.raises(ValueError):
        O.decode_fp32(L.codes, L.codebooks, L.scales[:4])
    with pytest.raises(ValueError):
        O.linear_ref_f64(L.codes, L.codebooks, L.scales, np.zeros((1, 32), np.float16))


# --------------------------------------------------------------------------
# Bit budget ("Memory footprint of AQLM-quantized models")


@pytest.mark.parametrize("scheme,out,n_in", [("2x8", 256, 512), ("1x16", 64, 128), ("2x8", 4096, 11008)])
def test_bit_budget_equals_stored_bytes(scheme, out, n_in):
    M, B, g, _ = synth.SCHEMES[scheme]
    L = synth.make_layer(scheme, out, n_in) if out * n_in <= 1 << 20 else None
    code_bytes = out * (n_in // g) * M * (B // 8)
    cb_bytes = M * (1 << B) * g * 2
    sc_bytes = out * 2
    if L is not None:
        assert (L.codes.nbytes, L.codebooks.nbytes, L.scales.nbytes) == (code_bytes, cb_bytes, sc_bytes)
    bpw = O.bits_per_weight(M, B, g, out, n_in)
    assert bpw == pytest.approx(8 * (code_bytes + cb_bytes + sc_bytes) / (out * n_in), rel=1e-15)


def test_bit_budget_pages_facts():
    facts = _load("pages_facts.json")
    f = facts["footprint_7b"]
    assert f["params"] * f["bits_per_param"] / 8 == f["aqlm_bytes"]
    assert f["fp16_bytes"] / f["aqlm_bytes"] == f["reduction"]
    bp = facts["budget_pairs_B8"]
    for M, g in bp["pairs"]:
        terms = O.bits_per_weight_terms(M, bp["B"], g, 4096, 4096)
        assert terms["codes"] == bp["bits"]
    names = facts["scheme_naming"]
    for scheme in ("1x16", "2x8"):
        M, B, g, _ = synth.SCHEMES[scheme]
        assert M * (1 << B) == names[scheme]["codewords_total"]
        assert O.bits_per_weight_terms(M, B, g, 4096, 4096)["codes"] == 2.0
    ffn = facts["llama2_70b_ffn"]
    d_in, d_out = ffn["d_in"], ffn["d_out"]
    for M, B, g in ((1, 16, 8), (2, 8, 8)):
        t = O.bits_per_weight_terms(M, B, g, d_out, d_in)
        assert t["scales"] < 0.01 * t["codes"]                 # scale term negligible
        assert t["codes"] > 10 * (t["codebooks"] + t["scales"])  # code term dominates
        assert abs(t["total"] - M * B / g) < 0.05               # ~ B*M/g
    small = O.bits_per_weight_terms(1, 8, 8, d_out, d_in)["codebooks"]
    large = O.bits_per_weight_terms(1, 16, 32, d_out, d_in)["codebooks"]
    assert large > 100 * small and large > 0.1  # codebooks matter only for large B and g
    t = O.bits_per_weight_terms(1, 16, 8, d_out, d_in)
    assert t["codebooks"] == pytest.approx(65536 * 8 * 16 / (d_out * d_in))
    assert t["scales"] == pytest.approx(16 / d_in)


# --------------------------------------------------------------------------
# Tolerance helper


def test_parity_errors_known_values():
    y_ref = np.array([[3.0, 4.0]])
    y = np.array([[3.0, 4.0 + 0.005]])
    rel, mx, ref_max = O.parity_errors(y, y_ref)
    assert rel == pytest.approx(0.001)
    assert mx == pytest.approx(0.005) and ref_max == 4.0
    assert O.within_tolerance(y, y_ref)
    assert not O.within_tolerance(np.array([[3.0, 4.1]]), y_ref)
