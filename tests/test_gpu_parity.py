"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars:
* decode: bit-exact fp16 weights;
* GEMV / GEMM: relative L2 error <= 1e-3 and max abs error <= 1e-2 * max|y_ref|
  over the compared outputs, y_ref from the oracle's fp32 decode and float64
  product.
Small cases and the full-size Llama-2-7B layers compare every output (the 7B
layers against the oracle computed in row chunks, plus a per-64-row-block
check, tests/parity_util.py), in the launch configuration the benchmark times.
The 70B layers compare every GEMV output too; only the 70B decode keeps
sampled rows (its W16 is 470 MB on the host).
"""
import numpy as np
import pytest
import torch

import extreme_weight_quantization_amd as E
from extreme_weight_quantization_amd import synth
from oracle import aqlm_oracle as O
from parity_util import assert_close_all, decode_full_bits, ref_full

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS_FRAC = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X")
    E.load_library()
    torch.cuda.init()


def dev(layer):
    codes = torch.from_numpy(layer.codes).cuda()
    cb = torch.from_numpy(layer.codebooks).cuda()
    s = torch.from_numpy(layer.scales).cuda()
    x = torch.from_numpy(layer.x).cuda()
    return codes, cb, s, x


def assert_close(y, y_ref, what=""):
    rel, mx, ref_max = O.parity_errors(y, y_ref)
    assert np.isfinite(rel), what
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC * ref_max, f"{what}: max abs {mx:.3e} > 1e-2 * {ref_max:.3e}"


def sample_rows(out, n=96, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(out, size=min(n, out), replace=False).tolist())
    rows |= {0, out - 1, min(15, out - 1), min(16, out - 1)}
    return np.array(sorted(rows), dtype=np.int64)


# --------------------------------------------------------------------------
# Decode: bit-exact


def check_decode(layer, rows=None):
    codes, cb, s, _ = dev(layer)
    w = E.aqlm_linear_decode(codes, cb, s)
    torch.cuda.synchronize()
    got = w.cpu().numpy()
    if rows is None:
        want = O.decode_fp16(layer.codes, layer.codebooks, layer.scales)
    else:
        want = O.decode_fp16(layer.codes, layer.codebooks, layer.scales, rows=rows)
        got = got[rows]
    diff = np.nonzero(got.view(np.uint16) != want.view(np.uint16))
    assert diff[0].size == 0, f"{diff[0].size} fp16 bit mismatches, first at {diff[0][0]},{diff[1][0]}"


@pytest.mark.parametrize("scheme,out,n_in", [
    ("2x8", 256, 512),      # tiny config, seed 0
    ("1x16", 256, 512),
    ("2x8", 33, 72),        # ragged: out not a multiple of 16, in % 64 != 0
    ("1x16", 17, 8),        # one group per row
    ("2x8", 1, 4096),
    ("1x16", 100, 4160),
])
def test_decode_bit_exact_small(scheme, out, n_in):
    check_decode(synth.make_layer(scheme, out, n_in, seed=0))


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
def test_decode_bit_exact_adversarial(scheme):
    L = synth.make_layer(scheme, 64, 256, seed=1)
    L.codebooks = synth.adversarial_codebooks(scheme, seed=1)
    M, B = L.M, L.B
    # extreme codes 0 and 2^B - 1, and the special entries 1..3
    rng = np.random.default_rng(5)
    special = np.array([0, (1 << B) - 1, 1, 2, 3])
    pick = rng.integers(0, len(special), size=L.codes.shape)
    if B == 8:
        L.codes = special[pick].astype(np.uint8)
    else:
        L.codes = special[pick].astype(np.uint16).view(np.int16)
    L.scales[:8] = np.array([1.0, -1.0, 0.5, 1.5, 2.0 ** -10, 1024.0, 0.0, -0.0], np.float16)
    check_decode(L)


@pytest.mark.parametrize("scheme,shape", [(s, sh) for s in ("2x8", "1x16") for sh in synth.LLAMA2_7B_SHAPES])
def test_decode_bit_exact_7b(scheme, shape):
    """Every weight of the full layer, bit for bit."""
    out, n_in = shape
    L = synth.make_layer(scheme, out, n_in, seed=0)
    codes, cb, s, _ = dev(L)
    got = E.aqlm_linear_decode(codes, cb, s).cpu().numpy().view(np.uint16)
    diff = np.nonzero(got != decode_full_bits(L))
    assert diff[0].size == 0, f"{diff[0].size} fp16 bit mismatches, first at {diff[0][0]},{diff[1][0]}"


def test_decode_bit_exact_70b_sampled():
    """28672 x 8192: sampled rows (the whole W16 would take 470 MB of host memory twice)."""
    L = synth.make_layer("1x16", 28672, 8192, seed=0)
    check_decode(L, rows=sample_rows(28672, 512))


def test_decode_deterministic():
    L = synth.make_layer("2x8", 512, 1024, seed=3)
    codes, cb, s, _ = dev(L)
    a = E.aqlm_linear_decode(codes, cb, s).cpu()
    b = E.aqlm_linear_decode(codes, cb, s).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------------------
# GEMV


def run_gemv(layer):
    codes, cb, s, x = dev(layer)
    y = E.aqlm_linear_gemv(codes, cb, s, x)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("out,n_in,batch", [
    (256, 512, 1),      # tiny config
    (100, 520, 3),      # ragged rows, partial slab, unaligned code rows
    (48, 4160, 16),     # partial last slab, aligned code rows
    (1, 8, 1),          # smallest layer
    (300, 2048, 7),
    (16, 16384, 2),     # wide row: many slabs per wave
    (4096 + 8, 256, 4), # many row tiles per workgroup
    (100, 520, 12),     # 16-row x stage: ragged rows, unaligned code rows
    (72, 4104, 8),      # 8-row x stage at its largest batch, a partial last slab
    (72, 4104, 9),      # 16-row x stage at its smallest batch
    (33, 4160, 16),     # aligned code rows, partial last slab, ragged row tile
])
def test_gemv_small(scheme, out, n_in, batch):
    L = synth.make_layer(scheme, out, n_in, batch=batch, seed=0)
    y = run_gemv(L)
    y_ref = O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
    assert_close(y, y_ref, f"{scheme} {out}x{n_in} b{batch}")


@pytest.mark.parametrize("out,n_in,batch", [
    (33, 4160, 1),      # 16 whole slabs and a ragged one, ragged row tile
    (33, 4160, 2),
    (4104, 256, 2),     # one slab: 16 waves split the row tiles, no slab parts
    (4104, 320, 1),     # a ragged second slab is all that one slab part holds
    (100, 192, 1),      # no whole slab at all
    (20000, 512, 1),    # several row tiles per wave in turn
    (70000, 256, 2),    # 18 row tiles per workgroup
    (64, 28672, 2),     # long slab ranges: 7 slabs a wave
])
def test_gemv_2x8_batch_1_2_every_output(out, n_in, batch):
    """The 2x8 product at batch 1-2 over 64-aligned inputs (codes and x streamed, the
    ragged last slab handled apart from the whole ones), every output against the oracle."""
    L = synth.make_layer("2x8", out, n_in, batch=batch, seed=out + n_in)
    y = run_gemv(L)
    assert_close_all(y, ref_full(L), f"2x8 {out}x{n_in} b{batch}")


def _random_2x8_stream_cases(n=8, seed=29):
    """Seeded shapes for the batch 1-2 2x8 product: rows 8000-20000, inputs 64-aligned with and
    without a ragged last slab; each gives a wave two or more slab steps (the streaming kernel),
    with 2-5 row tiles per workgroup."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(8000, 20000)), int(rng.choice([8192, 8256, 12288, 12352])), int(rng.integers(1, 3)))
            for _ in range(n)]


@pytest.mark.parametrize("out,n_in,batch", _random_2x8_stream_cases())
def test_gemv_2x8_batch_1_2_random_shapes_every_output(out, n_in, batch):
    L = synth.make_layer("2x8", out, n_in, batch=batch, seed=out ^ n_in)
    assert_close_all(run_gemv(L), ref_full(L), f"2x8 {out}x{n_in} b{batch}")


@pytest.mark.parametrize("out,n_in,batch", [
    (9000, 8192, 3),    # three row tiles a workgroup, two slabs a wave
    (9000, 8256, 4),    # a ragged last slab at batch 4
    (20000, 4096, 4),   # one slab a wave, five row tiles a workgroup
    (8200, 12288, 3),   # the largest x that fits the LDS at batch 3
])
def test_gemv_2x8_batch_3_4_stream_every_output(out, n_in, batch):
    """The 2x8 product at batch 3-4 on layers that give a wave four or more slab steps (the
    streaming kernel, x rows padded apart in LDS), every output against the oracle."""
    L = synth.make_layer("2x8", out, n_in, batch=batch, seed=out + batch)
    assert_close_all(run_gemv(L), ref_full(L), f"2x8 {out}x{n_in} b{batch}")


@pytest.mark.parametrize("outs,n_in,batch", [((9000, 5000, 13000), 8192, 1), ((12000, 700), 12288, 2),
                                             ((9000, 1024, 9000), 8192, 4)])
def test_gemv_2x8_fused_stream_every_output(outs, n_in, batch):
    """Fused layers on the streaming kernel (the layers' workgroups dealt by size): bit-identical to
    separate calls, every output of every layer against the oracle."""
    x = synth.make_activations(n_in, batch, seed=5)
    xd = torch.from_numpy(x).cuda()
    layers, hosts = [], []
    for li, out in enumerate(outs):
        L = synth.make_layer("2x8", out, n_in, batch=batch, seed=40 + li)
        L.x = x
        layers.append(tuple(torch.from_numpy(a).cuda() for a in (L.codes, L.codebooks, L.scales)))
        hosts.append(L)
    ys = E.aqlm_linear_gemv_fused(layers, xd)
    torch.cuda.synchronize()
    for (c, cb, sc), y, L in zip(layers, ys, hosts):
        y_sep = E.aqlm_linear_gemv(c, cb, sc, xd)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_sep.view(torch.int16))
        assert_close_all(y.cpu().numpy(), ref_full(L), f"fused {L.codes.shape[0]}x{n_in} b{batch}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("batch", [3, 16])
def test_gemv_several_passes_and_slabs(scheme, batch):
    """8200 rows: workgroups run a second pass of row tiles, and 545 groups make
    two slabs for some waves, so a pass re-stages x after the previous pass's
    partial tiles were summed in the same LDS."""
    L = synth.make_layer(scheme, 8200, 4360, batch=batch, seed=batch)
    y = run_gemv(L)
    rows = np.unique(np.concatenate([sample_rows(8200, 48), np.arange(8184, 8200), np.arange(4096, 4112)]))
    assert_close(y[:, rows], O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, L.x, rows), f"{scheme} b{batch}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("big,small", [(8, 3), (16, 9)])
def test_gemv_stale_stage_rows_do_not_leak(scheme, big, small):
    """A call at a larger batch leaves NaN in the LDS rows of x that a following
    call at a smaller batch does not load; its outputs stay finite and right."""
    L = synth.make_layer(scheme, 512, 2048, batch=big, seed=7)
    L.x[small:] = np.nan
    codes, cb, s, x = dev(L)
    y_big = E.aqlm_linear_gemv(codes, cb, s, x)
    y = E.aqlm_linear_gemv(codes, cb, s, x[:small].contiguous()).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert torch.isnan(y_big[small:]).all()
    assert np.isfinite(y).all()
    assert_close(y, O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x[:small]), f"{scheme} b{small} after b{big}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
def test_gemv_every_batch_size(scheme):
    for batch in range(1, 17):
        L = synth.make_layer(scheme, 64, 512, batch=batch, seed=batch)
        assert_close(run_gemv(L), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), f"b{batch}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
def test_gemv_basis_vectors_exact(scheme):
    """Dyadic one-hot codebooks make every weight exact: x = e_k returns column k of W16 exactly."""
    M, B, g, _ = synth.SCHEMES[scheme]
    cb = np.zeros((M, 1 << B, g), np.float16)
    k = np.arange(1 << B)
    for m in range(M):
        cb[m, k, k % 8] = (2.0 ** -(m + 1)) * (((k >> 3) % 32) + 1) / 32
    L = synth.make_layer(scheme, 40, 128, batch=16, seed=2)
    L.codebooks = cb
    L.scales = np.random.default_rng(0).choice([0.5, 1.0, 1.5, 2.0], size=40).astype(np.float16)
    cols = [0, 1, 7, 8, 63, 64, 100, 127, 9, 17, 33, 50, 77, 90, 111, 126]
    L.x = np.zeros((16, 128), np.float16)
    for b, c in enumerate(cols):
        L.x[b, c] = 1
    y = run_gemv(L)
    w16 = O.decode_fp16(L.codes, L.codebooks, L.scales).astype(np.float64)
    np.testing.assert_array_equal(y, w16[:, cols].T)


@pytest.mark.parametrize("batch", [1, 16])
@pytest.mark.parametrize("shape", synth.LLAMA2_7B_SHAPES)
def test_gemv_7b_1x16(shape, batch):
    out, n_in = shape
    L = synth.make_layer("1x16", out, n_in, batch=batch, seed=0)
    assert_close_all(run_gemv(L), ref_full(L), str(shape))


@pytest.mark.parametrize("batch", [1, 4, 16])
@pytest.mark.parametrize("shape", synth.LLAMA2_7B_SHAPES)
def test_gemv_7b_2x8(shape, batch):
    out, n_in = shape
    L = synth.make_layer("2x8", out, n_in, batch=batch, seed=0)
    assert_close_all(run_gemv(L), ref_full(L), str(shape))


@pytest.mark.parametrize("shape", synth.LLAMA2_70B_SHAPES)
def test_gemv_70b_1x16(shape):
    out, n_in = shape
    L = synth.make_layer("1x16", out, n_in, batch=1, seed=0)
    assert_close_all(run_gemv(L), ref_full(L), str(shape))


def test_gemv_accepts_given_output_and_stream():
    L = synth.make_layer("2x8", 64, 256, batch=2, seed=4)
    codes, cb, s, x = dev(L)
    y = torch.full((2, 64), float("nan"), dtype=torch.float16, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        E.aqlm_linear_gemv(codes, cb, s, x, y)
    st.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64),
                 O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x))


# --------------------------------------------------------------------------
# Fused GEMV: several layers sharing x in one launch


def run_fused(layers, x):
    dl = [dev(L)[:3] for L in layers]
    xd = torch.from_numpy(x).cuda()
    ys = E.aqlm_linear_gemv_fused(dl, xd)
    torch.cuda.synchronize()
    sep = [E.aqlm_linear_gemv(c, cb, s, xd) for (c, cb, s) in dl]
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], [y.cpu().numpy() for y in sep]


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("outs,n_in,batch", [
    ((4096, 4096, 4096), 4096, 1),        # q, k, v of a 7B attention block
    ((4096, 4096, 4096), 4096, 16),
    ((4096,) * 4, 11008, 16),             # 64 workgroups a layer: two passes of three slabs a wave
    ((11008, 11008), 4096, 4),            # gate, up of a 7B MLP
    ((100, 4096, 37, 1000), 520, 3),      # ragged rows and in, uneven layers
    ((100, 4096, 37, 1000), 576, 1),      # ragged rows and last slab, 64-aligned in
    ((28672, 28672), 8192, 2),            # 70B gate, up: 14 row tiles per workgroup
    ((28672, 28672), 8192, 4),            # the same at batch 4: streamed, one launch per layer (LDS)
    ((8192, 1024, 1024), 8192, 3),        # 70B q, k, v at batch 3: q streamed, k and v not
    ((16,) * 8, 256, 1),                  # the most layers one call takes
])
def test_gemv_fused_matches_separate_and_oracle(scheme, outs, n_in, batch):
    layers = [synth.make_layer(scheme, o, n_in, batch=batch, seed=10 + i) for i, o in enumerate(outs)]
    x = layers[0].x
    fused, sep = run_fused(layers, x)
    for i, (L, yf, ys) in enumerate(zip(layers, fused, sep)):
        np.testing.assert_array_equal(yf.view(np.uint16), ys.view(np.uint16), err_msg=f"layer {i}")
        rows = sample_rows(L.codes.shape[0], 32)
        ref = O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, x, rows)
        assert_close(yf.astype(np.float64)[:, rows], ref, f"{scheme} fused layer {i}")


def test_gemv_fused_skips_empty_layers():
    a = synth.make_layer("2x8", 300, 512, batch=2, seed=1)
    b = synth.make_layer("2x8", 64, 512, batch=2, seed=2)
    xd = torch.from_numpy(a.x).cuda()
    empty = (torch.zeros((0, 64, 2), dtype=torch.uint8, device="cuda"),
             torch.from_numpy(b.codebooks).cuda(), torch.zeros(0, dtype=torch.float16, device="cuda"))
    ys = E.aqlm_linear_gemv_fused([dev(a)[:3], empty, dev(b)[:3]], xd)
    torch.cuda.synchronize()
    assert ys[1].shape == (2, 0)
    for L, y in ((a, ys[0]), (b, ys[2])):
        assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(L.codes, L.codebooks, L.scales, a.x), "skip")


# --------------------------------------------------------------------------
# GEMM


def run_gemm(layer):
    codes, cb, s, x = dev(layer)
    y = E.aqlm_linear_gemm(codes, cb, s, x)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("out,n_in,batch", [
    (256, 512, 1),
    (100, 520, 5),      # ragged everything
    (300, 4160, 130),   # several tiles, ragged tails
    (128, 256, 256),
    (17, 8, 3),
    (200, 64, 70),      # a single k-step
    (1000, 1024, 513),  # pipelined path: several row and token tiles, ragged
    (129, 64, 257),     # pipelined path: one k-step, rows not a multiple of 8, a second token tile
    (70, 1088, 300),    # pipelined path: 17 k-steps (the code ring wraps), ragged rows and tokens
])
def test_gemm_small(scheme, out, n_in, batch):
    L = synth.make_layer(scheme, out, n_in, batch=batch, seed=0)
    y = run_gemm(L)
    assert_close(y, O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), f"{scheme} {out}x{n_in} T{batch}")


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("n_in", [136, 192])
def test_gemm_basis_exact(scheme, n_in):
    """X = identity rows: Y equals W16 transposed exactly with dyadic one-hot codebooks.

    in = 136 runs the general kernel, in = 192 (a multiple of 64) the 2x8 pipelined one."""
    M, B, g, _ = synth.SCHEMES[scheme]
    cb = np.zeros((M, 1 << B, g), np.float16)
    k = np.arange(1 << B)
    for m in range(M):
        cb[m, k, k % 8] = (2.0 ** -(m + 1)) * (((k >> 3) % 32) + 1) / 32
    L = synth.make_layer(scheme, 72, n_in, batch=n_in, seed=3)
    L.codebooks = cb
    L.scales = np.random.default_rng(1).choice([0.5, 1.0, 2.0], size=72).astype(np.float16)
    L.x = np.eye(n_in, dtype=np.float16)
    y = run_gemm(L)
    np.testing.assert_array_equal(y, O.decode_fp16(L.codes, L.codebooks, L.scales).astype(np.float64).T)


@pytest.mark.parametrize("scheme", ["2x8", "1x16"])
@pytest.mark.parametrize("shape", synth.LLAMA2_7B_SHAPES)
def test_gemm_prefill_7b(scheme, shape):
    """All 2048 tokens x every output row."""
    out, n_in = shape
    L = synth.make_layer(scheme, out, n_in, batch=2048, seed=0)
    assert_close_all(run_gemm(L), ref_full(L), f"{scheme} {shape}")


def test_gemm_matches_gemv_for_small_batch():
    L = synth.make_layer("2x8", 512, 1024, batch=8, seed=6)
    a, b = run_gemm(L), run_gemv(L)
    assert_close(a, b, "gemm vs gemv")


# --------------------------------------------------------------------------
# Generic schemes: any (M, B, g), codes in whole bytes indexed by their low B bits

GENERIC = [(1, 8, 4), (4, 8, 16), (8, 8, 32), (3, 5, 8), (1, 12, 4), (2, 16, 32), (1, 12, 1), (3, 5, 2),
           (2, 8, 16), (1, 16, 8 // 2)]


def junk_high_bits(codes, B, seed=7):
    """Random bits in the unused high part of every stored code (the index is the low B bits)."""
    rng = np.random.default_rng(seed)
    bits = 8 if codes.dtype == np.uint8 else 16
    if B == bits:
        return codes.copy()
    u = codes.view(np.uint8 if bits == 8 else np.uint16).astype(np.int64)
    out = (u | (rng.integers(0, 1 << (bits - B), size=u.shape) << B)).astype(np.uint8 if bits == 8 else np.uint16)
    return out if bits == 8 else out.view(np.int16)


def gdev(L, codes):
    return (torch.from_numpy(codes).cuda(), torch.from_numpy(L.codebooks).cuda(),
            torch.from_numpy(L.scales).cuda(), torch.from_numpy(L.x).cuda())


@pytest.mark.parametrize("M,B,g", GENERIC)
def test_generic_decode_bit_exact(M, B, g):
    L = synth.make_layer_mbg(M, B, g, 67, g * 37, seed=M + B + g)
    codes = junk_high_bits(L.codes, B)
    c, cb, s, _ = gdev(L, codes)
    w = E.aqlm_linear_decode(c, cb, s)
    torch.cuda.synchronize()
    want = O.decode_fp16(codes, L.codebooks, L.scales)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M,B,g", [(1, 8, 4), (3, 5, 2), (1, 12, 1), (1, 16, 4), (1, 12, 4)])
def test_generic_decode_bit_exact_whole_pieces(M, B, g):
    """g < 8 with in % 8 == 0: a thread decodes 8/g groups of one row into one 16-byte store."""
    L = synth.make_layer_mbg(M, B, g, 67, 8 * 41, seed=M + B + g + 1)
    codes = junk_high_bits(L.codes, B)
    c, cb, s, _ = gdev(L, codes)
    w = E.aqlm_linear_decode(c, cb, s)
    torch.cuda.synchronize()
    want = O.decode_fp16(codes, L.codebooks, L.scales)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M,B,g", GENERIC)
@pytest.mark.parametrize("batch", [1, 5, 16])
def test_generic_gemv(M, B, g, batch):
    L = synth.make_layer_mbg(M, B, g, 131, g * 45, batch=batch, seed=3 * M + B)
    codes = junk_high_bits(L.codes, B)
    c, cb, s, x = gdev(L, codes)
    y = E.aqlm_linear_gemv(c, cb, s, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(codes, L.codebooks, L.scales, L.x),
                 f"gemv {M}x{B}g{g} T{batch}")


# The other 2-bit schemes with B = 8 (g = 4 M).  Their GEMV runs the 2x8 kernel when
# in % 8 == 0 (1x8 g4 and 4x8 g16 at every batch with direct x, 8-row and 16-row stages;
# 8x8 g32 above batch 8, with direct x), else the general one.
B8_FAMILY = [(1, 8, 4), (4, 8, 16), (8, 8, 32)]


@pytest.mark.parametrize("M,B,g", B8_FAMILY)
@pytest.mark.parametrize("out,n_in,batch", [
    (300, 4096, 1),     # direct x loads, one slab per wave
    (300, 4096, 2),
    (72, 4160, 3),      # 8-row x stage, partial last slab, aligned code rows
    (72, 4160, 8),
    (100, 1056, 9),     # 16-row x stage, unaligned code rows
    (33, 4160, 16),     # ragged row tile
    (4104, 512, 4),     # many row tiles per workgroup
    (16, 16384, 1),     # many slabs per wave
])
def test_gemv_b8_family(M, B, g, out, n_in, batch):
    L = synth.make_layer_mbg(M, B, g, out, n_in, batch=batch, seed=out + batch + M)
    c, cb, s, x = gdev(L, L.codes)
    y = E.aqlm_linear_gemv(c, cb, s, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x),
                 f"gemv {M}x{B}g{g} {out}x{n_in} T{batch}")


@pytest.mark.parametrize("M,B,g", B8_FAMILY)
@pytest.mark.parametrize("shape,batch", [((4096, 11008), 16), ((11008, 4096), 1), ((4096, 4096), 4)])
def test_gemv_b8_family_7b(M, B, g, shape, batch):
    out, n_in = shape
    L = synth.make_layer_mbg(M, B, g, out, n_in, batch=batch, seed=M)
    c, cb, s, x = gdev(L, L.codes)
    y = E.aqlm_linear_gemv(c, cb, s, x).cpu().numpy().astype(np.float64)
    assert_close_all(y, ref_full(L), f"gemv {M}x{B}g{g} {shape} T{batch}")


def test_gemv_1x8g4_unaligned_in_runs_the_general_kernel():
    """in % 8 != 0 (in = 4 * odd): 1x8 g4 falls back to the general kernel."""
    L = synth.make_layer_mbg(1, 8, 4, 200, 4 * 1027, batch=3, seed=11)
    c, cb, s, x = gdev(L, L.codes)
    y = E.aqlm_linear_gemv(c, cb, s, x).cpu().numpy().astype(np.float64)
    assert_close(y, O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x), "1x8g4 in=4108")


@pytest.mark.parametrize("M,B,g", B8_FAMILY)
@pytest.mark.parametrize("batch", [5, 16])
def test_gemv_b8_family_fused(M, B, g, batch):
    """The fused entry point (one launch, or one per layer on the general kernel) equals separate calls."""
    layers = [synth.make_layer_mbg(M, B, g, o, 2048, batch=batch, seed=20 + i) for i, o in enumerate((300, 4096, 100))]
    xd = torch.from_numpy(layers[0].x).cuda()
    dl = [gdev(L, L.codes)[:3] for L in layers]
    ys = E.aqlm_linear_gemv_fused(dl, xd)
    sep = [E.aqlm_linear_gemv(c, cb, s, xd) for (c, cb, s) in dl]
    torch.cuda.synchronize()
    for i, (L, yf, ys1) in enumerate(zip(layers, ys, sep)):
        np.testing.assert_array_equal(yf.cpu().numpy().view(np.uint16), ys1.cpu().numpy().view(np.uint16))
        rows = sample_rows(L.codes.shape[0], 32)
        assert_close(yf.cpu().numpy().astype(np.float64)[:, rows],
                     O.linear_ref_rows_f64(L.codes, L.codebooks, L.scales, layers[0].x, rows), f"fused layer {i}")


@pytest.mark.parametrize("M,B,g", GENERIC)
@pytest.mark.parametrize("out,n_grp,batch", [(200, 37, 130), (64, 8, 3)])
def test_generic_gemm(M, B, g, out, n_grp, batch):
    """Several tiles with ragged rows, tokens and inputs (in % 8 != 0 when g < 8 and n_grp is odd)."""
    L = synth.make_layer_mbg(M, B, g, out, g * n_grp, batch=batch, seed=5 * M + B + g)
    codes = junk_high_bits(L.codes, B)
    c, cb, s, x = gdev(L, codes)
    y = E.aqlm_linear_gemm(c, cb, s, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(codes, L.codebooks, L.scales, L.x),
                 f"gemm {M}x{B}g{g} {out}x{g * n_grp} T{batch}")


@pytest.mark.parametrize("out,n_in,batch", [(300, 1088, 130), (129, 64, 257), (64, 2048, 1)])
def test_gemm_1x8g4_pipeline(out, n_in, batch):
    """1x8 g4 with in % 64 == 0 runs the pipelined 2x8 prefill: ragged rows and tokens, a
    single k-step, a single token."""
    L = synth.make_layer_mbg(1, 8, 4, out, n_in, batch=batch, seed=out + batch)
    c, cb, s, x = gdev(L, L.codes)
    y = E.aqlm_linear_gemm(c, cb, s, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x),
                 f"1x8g4 gemm {out}x{n_in} T{batch}")


@pytest.mark.parametrize("out,n_in,batch", [(300, 1088, 130), (129, 64, 257), (64, 2048, 1), (4104, 4096, 300)])
def test_gemm_4x8g16_pipeline(out, n_in, batch):
    """4x8 g16 with in % 64 == 0 runs the pipelined 2x8 prefill with two X stages: ragged rows
    and tokens, a single k-step, a single token, many row tiles; every output."""
    L = synth.make_layer_mbg(4, 8, 16, out, n_in, batch=batch, seed=out + 3 * batch)
    c, cb, s, x = gdev(L, L.codes)
    y = E.aqlm_linear_gemm(c, cb, s, x)
    torch.cuda.synchronize()
    assert_close_all(y.cpu().numpy(), ref_full(L), f"4x8g16 gemm {out}x{n_in} T{batch}")


@pytest.mark.parametrize("M,B,g", [(4, 8, 16), (1, 8, 4), (3, 5, 2)])
def test_generic_exact_on_identity(M, B, g):
    """Dyadic one-hot codebooks and X = I: GEMM and GEMV return W16 columns exactly."""
    K = 1 << B
    k = np.arange(K)
    cb = np.zeros((M, K, g), np.float16)
    for m in range(M):
        cb[m, k, k % g] = (2.0 ** -(m + 1)) * ((k // g) % 32 + 1) / 32
    n_in = 16 * g if g >= 8 else 64
    L = synth.make_layer_mbg(M, B, g, 40, n_in, batch=n_in, seed=9)
    L.codebooks = cb
    L.scales = np.random.default_rng(2).choice([0.5, 1.0, 2.0], size=40).astype(np.float16)
    L.x = np.eye(n_in, dtype=np.float16)
    c, cbd, s, x = gdev(L, L.codes)
    want = O.decode_fp16(L.codes, cb, L.scales).astype(np.float64).T
    y = E.aqlm_linear_gemm(c, cbd, s, x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), want)
    y1 = E.aqlm_linear_gemv(c, cbd, s, x[:16].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y1.cpu().numpy().astype(np.float64), want[:16])


@pytest.mark.parametrize("M,B,g", [(4, 8, 16), (8, 8, 32), (1, 8, 4), (2, 12, 8)])
def test_generic_full_size_7b(M, B, g):
    """4096x4096 at 2 bits per weight, every output: decode bit-exact, GEMV b1, GEMM 2048 tokens."""
    L = synth.make_layer_mbg(M, B, g, 4096, 4096, batch=1, seed=0)
    c, cb, s, x = gdev(L, L.codes)
    w = E.aqlm_linear_decode(c, cb, s)
    y = E.aqlm_linear_gemv(c, cb, s, x)
    xs_h = synth.make_activations(4096, 2048, seed=1)
    xs = torch.from_numpy(xs_h).cuda()
    yg = E.aqlm_linear_gemm(c, cb, s, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), decode_full_bits(L))
    assert_close_all(y.cpu().numpy(), ref_full(L), "gemv")
    assert_close_all(yg.cpu().numpy(), ref_full(L, xs_h), "gemm")


# --------------------------------------------------------------------------
# Greedy residual encoder and residual k-means (bit-exact against the oracle)


def weights(out, n_in, seed, sigma=0.05):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, sigma, size=(out, n_in)).astype(np.float16)
    s = rng.uniform(0.5, 1.5, size=out).astype(np.float16) * np.float16(sigma)
    return w, s.astype(np.float16)


ENC_SCHEMES = [(2, 8, 8), (1, 16, 8), (4, 8, 16), (1, 12, 4), (3, 5, 2), (8, 8, 32)]


@pytest.mark.parametrize("M,B,g", ENC_SCHEMES)
def test_encode_greedy_bit_exact(M, B, g):
    out, n_in = (24, 4 * g) if B > 12 else (67, 6 * g)
    w, s = weights(out, n_in, seed=M + B)
    cb = np.random.default_rng(1).normal(0, 1, size=(M, 1 << B, g)).astype(np.float16)
    codes = E.aqlm_encode_greedy(torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), torch.from_numpy(cb).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), O.encode_greedy(w, s, cb))


def test_encode_greedy_recovers_planted_codes():
    L = synth.make_layer_mbg(1, 8, 8, 300, 512, seed=4, sigma=1.0)
    w = O.decode_fp16(L.codes, L.codebooks, L.scales)
    codes = E.aqlm_encode_greedy(torch.from_numpy(w).cuda(), torch.from_numpy(L.scales).cuda(),
                                 torch.from_numpy(L.codebooks).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), L.codes)


@pytest.mark.parametrize("M,B,g,out,n_in,iters", [
    (2, 8, 8, 64, 256, 3),
    (1, 8, 4, 40, 64, 4),
    (3, 5, 8, 33, 96, 2),
    (1, 12, 4, 64, 64, 2),
])
def test_kmeans_init_bit_exact(M, B, g, out, n_in, iters):
    w, s = weights(out, n_in, seed=out)
    N = out * n_in // g
    rng = np.random.default_rng(2)
    seeds = np.stack([rng.choice(N, 1 << B, replace=(1 << B) > N) for _ in range(M)]).astype(np.int64)
    cb, codes = E.aqlm_kmeans_init(torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(),
                                   torch.from_numpy(seeds).cuda(), B, g, iters)
    torch.cuda.synchronize()
    cb_ref, codes_ref = O.kmeans_residual_init(w, s, seeds, M, B, g, iters)
    np.testing.assert_array_equal(cb.cpu().numpy().view(np.uint16), cb_ref.view(np.uint16))
    np.testing.assert_array_equal(codes.cpu().numpy(), codes_ref)


@pytest.mark.parametrize("B,g", [(11, 8), (12, 4)])
def test_encode_greedy_ties_across_chunks(B, g):
    """Codebooks made of repeated 1024-codeword blocks: equal distances in different 1024-codeword
    chunks go to the lowest index, as in the oracle (codes all below 1024, bit-identical)."""
    rng = np.random.default_rng(B)
    base = rng.normal(0, 1, size=(1024, g)).astype(np.float16)
    cb = np.concatenate([base] * ((1 << B) // 1024))[None]
    w, s = weights(40, 24 * g, seed=B)
    codes = E.aqlm_encode_greedy(torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), torch.from_numpy(cb).cuda())
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    np.testing.assert_array_equal(got, O.encode_greedy(w, s, cb))
    assert int(got.view(np.uint16).max()) < 1024


def test_kmeans_init_bit_exact_members_near_the_fixed_point_grid():
    """Weights that are small multiples of 2^-24 (fp16 subnormals) over scales 0.5 .. 4: the targets
    fall on and between multiples of 2^-24, halves included, so the centroid sums exercise the
    rounding to the fixed-point grid (halves to even); codebooks and codes equal the oracle's."""
    rng = np.random.default_rng(21)
    out, n_in, g, B, M = 48, 64, 4, 6, 2
    w = (rng.integers(-6, 7, size=(out, n_in)) * 2.0 ** -24).astype(np.float16)
    s = rng.choice([0.5, 0.75, 1.5, 3.0, 4.0], size=out).astype(np.float16)
    N = out * n_in // g
    seeds = np.stack([rng.choice(N, 1 << B, replace=False) for _ in range(M)]).astype(np.int64)
    cb, codes = E.aqlm_kmeans_init(torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(),
                                   torch.from_numpy(seeds).cuda(), B, g, 3)
    torch.cuda.synchronize()
    cb_ref, codes_ref = O.kmeans_residual_init(w, s, seeds, M, B, g, 3)
    np.testing.assert_array_equal(cb.cpu().numpy().view(np.uint16), cb_ref.view(np.uint16))
    np.testing.assert_array_equal(codes.cpu().numpy(), codes_ref)


def test_kmeans_init_out_of_range_targets_give_nan_codebooks():
    """Scales of 2^-14 make |W/s| reach 2^13, above the exact-sum bound 2^29 / n_groups (2^29 / 2^17
    groups = 2^12): the codebooks come out NaN and the codes 0 instead of wrapped sums.  The same
    weights with unit scales stay in range and match the oracle."""
    rng = np.random.default_rng(22)
    out, n_in, B, g = 2048, 512, 6, 8          # 2^17 groups
    w = (rng.normal(0, 0.25, size=(out, n_in))).astype(np.float16)
    seeds = rng.choice(out * n_in // g, (1, 1 << B), replace=False).astype(np.int64)
    tiny = np.full(out, 2.0 ** -14, np.float16)
    cb, codes = E.aqlm_kmeans_init(torch.from_numpy(w).cuda(), torch.from_numpy(tiny).cuda(),
                                   torch.from_numpy(seeds).cuda(), B, g, 2)
    torch.cuda.synchronize()
    assert np.isnan(cb.cpu().numpy().astype(np.float32)).all()
    assert not codes.cpu().numpy().any()
    ones = np.ones(out, np.float16)
    cb, codes = E.aqlm_kmeans_init(torch.from_numpy(w).cuda(), torch.from_numpy(ones).cuda(),
                                   torch.from_numpy(seeds).cuda(), B, g, 2)
    torch.cuda.synchronize()
    cb_ref, codes_ref = O.kmeans_residual_init(w, ones, seeds, 1, B, g, 2)
    np.testing.assert_array_equal(cb.cpu().numpy().view(np.uint16), cb_ref.view(np.uint16))
    np.testing.assert_array_equal(codes.cpu().numpy(), codes_ref)


def test_encode_and_kmeans_full_size_2x8():
    """4096x4096 weights: encoder codes on sampled rows equal the oracle's; the k-means codes are the
    greedy encoding against the k-means codebooks (checked on sampled rows)."""
    w, s = weights(4096, 4096, seed=0)
    wd, sd = torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda()
    cb = np.random.default_rng(3).normal(0, 1, size=(2, 256, 8)).astype(np.float16)
    codes = E.aqlm_encode_greedy(wd, sd, torch.from_numpy(cb).cuda())
    N = 4096 * 512
    seeds = np.stack([np.random.default_rng(5 + m).choice(N, 256, replace=False) for m in range(2)])
    kcb, kcodes = E.aqlm_kmeans_init(wd, sd, torch.from_numpy(seeds).cuda(), 8, 8, 2)
    torch.cuda.synchronize()
    rows = sample_rows(4096, 24)
    np.testing.assert_array_equal(codes.cpu().numpy()[rows], O.encode_greedy(w[rows], s[rows], cb))
    kcb = kcb.cpu().numpy()
    np.testing.assert_array_equal(kcodes.cpu().numpy()[rows], O.encode_greedy(w[rows], s[rows], kcb))
    # the k-means codebooks reconstruct the layer better than random codebooks of the same spread
    err_km = np.abs(O.decode_fp32(kcodes.cpu().numpy()[rows], kcb, s[rows]) - w[rows].astype(np.float32)).mean()
    err_rand = np.abs(O.decode_fp32(codes.cpu().numpy()[rows], cb, s[rows]) - w[rows].astype(np.float32)).mean()
    assert err_km < err_rand


# --------------------------------------------------------------------------
# Errors through the binding


def test_binding_errors_on_gpu():
    L = synth.make_layer("2x8", 64, 256, batch=1, seed=0)
    codes, cb, s, x = dev(L)
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv(codes, cb[:, :100].contiguous(), s, x)      # 100 codewords: not 2^B
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv(codes, torch.zeros((2, 512, 8), dtype=torch.float16, device="cuda"), s, x)  # B = 9, uint8 codes
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv(codes, cb, s, torch.zeros((17, 256), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv(codes, cb, s, x[:, :128])
    y0 = E.aqlm_linear_gemm(codes, cb, s, torch.zeros((0, 256), dtype=torch.float16, device="cuda"))
    assert y0.shape == (0, 64)
    # shapes that would make a kernel read past a buffer are refused on the host, before any launch
    one_code = codes[:, :, :1].contiguous()                 # uint8 [out][G][1] with 2x8 codebooks
    for fn in (E.aqlm_linear_gemv, E.aqlm_linear_gemm, E.aqlm_linear_gemm_dequant):
        with pytest.raises(ValueError, match="codebooks"):
            fn(one_code, cb, s, x)
        with pytest.raises(ValueError, match="scales"):
            fn(codes, cb, s[:32].contiguous(), x)         # 32 scales for 64 rows
    with pytest.raises(ValueError, match="codebooks"):
        E.aqlm_linear_decode(one_code, cb, s)
    with pytest.raises(ValueError, match="scales"):
        E.aqlm_linear_decode(codes, cb, s[:63].contiguous())
    with pytest.raises(ValueError, match="scales"):
        E.aqlm_linear_gemv_fused([(codes, cb, s), (codes, cb, s[:10].contiguous())], x)
    with pytest.raises(ValueError, match="codebooks"):
        E.aqlm_linear_gemv_fused([(codes, cb, s), (one_code, cb, s)], x)
    L16 = synth.make_layer("1x16", 64, 256, batch=1, seed=1)
    c16, cb16, s16, x16 = dev(L16)
    lists = E.aqlm_lists_pack(c16)
    with pytest.raises(ValueError, match="scales"):
        E.aqlm_linear_gemv_lists(lists, cb16, s16[:8].contiguous(), x16)
    with pytest.raises(ValueError, match="scales"):
        E.aqlm_linear_gemv_lists_fused([(lists, cb16, s16[:8].contiguous())], x16)
    torch.cuda.synchronize()
