"""Plain, slow CPU oracle for the AQLM quantized linear layer y = W x.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call anything here.  It shares
no code with the HIP library and imports nothing from it; both sides receive
the same arrays from the seeded input generators.

Sources (cited by page title and section):

* "The AQLM Quantization Algorithm, Explained", section "What is Multi-Codebook
  Quantization (MCQ)?": a row of W (shape d_out x d_in, W.X convention) is cut
  into groups of g consecutive inputs; each group is approximated by the sum
  of M codewords, one from each of M codebooks of 2^B codewords of size g held
  at 16-bit precision; a group stores M indices of B bits; every output
  channel carries a learned scale.  Figure 2 (dequantization): the selected
  codewords are summed, then scaled, giving half-precision weights that the
  matrix product consumes.
* Same page, section "Memory footprint of AQLM-quantized models": the stored
  items are M codebooks of 2^B fp16 codewords of size g, d_out fp16 scales and
  M codes of B bits for each of the d_out*d_in/g groups; the average bits per
  parameter is taken per weight matrix.  The formula itself did not survive
  text extraction, so ``bits_per_weight`` re-derives it from those three
  listed items.
* Same page, section "Key AQLM quantization parameters": when the code term
  dominates, bits per parameter is about B*M/g; at B = 8 the pairs (M, g) =
  (1, 4), (2, 8), ..., (8, 32) all give 2 bits; a B that is not a multiple of
  8 leaves unused bits in the bytes that hold each code.

Readings where the pages are silent:

* group j of row i covers columns [j*g, (j+1)*g); codes are stored
  ``[d_out][d_in/g][M]``; codebooks ``[M][2^B][g]``; scales ``[d_out]``;
* a code is stored in whole bytes, uint8 for B <= 8 and int16 for
  9 <= B <= 16 (the "unused bits" note above); its codeword index is the low B
  bits of the stored pattern read as unsigned (a B=16 code in an int16 is
  0..65535, a B=8 code in a uint8 is its value, higher bits are ignored);
* the codewords are summed in fp32, codebook 0 first then m ascending, the
  running sum starting from codebook 0's codeword (not from +0.0), then
  multiplied by the fp32 scale; the fp16 weight is that fp32 value rounded to
  nearest-even with subnormals kept;
* the reference product uses the fp32 decoded weights widened to float64.

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, brute force on one-hot codebooks and facts the pages print.
"""
from __future__ import annotations

import math

import numpy as np

# The two named schemes at g = 8 ("Key AQLM quantization parameters": XBit-MxB
# naming, e.g. 2Bit-1x16).  The oracle itself decodes any (M, B, g) with
# M >= 1, 1 <= B <= 16, g >= 1.
SUPPORTED_SCHEMES = ((1, 16, 8), (2, 8, 8))


def _check_layer(codes, codebooks, scales):
    """Shape and dtype checks for one quantized layer; returns (M, B, g, out, in)."""
    if codebooks.dtype != np.float16 or codebooks.ndim != 3:
        raise ValueError("codebooks must be float16 [M][2^B][g]")
    M, K, g = codebooks.shape
    B = int(round(math.log2(K))) if K > 0 else -1
    if K <= 0 or (1 << B) != K or B < 1:
        raise ValueError("codebook size must be a power of two >= 2")
    if M < 1 or g < 1:
        raise ValueError("need M >= 1 codebooks of g >= 1 entries")
    if codes.ndim != 3 or codes.shape[2] != M:
        raise ValueError("codes must be [out][in/g][M]")
    if B <= 8:
        if codes.dtype != np.uint8:
            raise ValueError("B <= 8 codes must be uint8")
    elif B <= 16:
        if codes.dtype not in (np.int16, np.uint16):
            raise ValueError("9 <= B <= 16 codes must be int16 (bit pattern) or uint16")
    else:
        raise ValueError("B > 16 not representable")
    out, G, _ = codes.shape
    if scales.dtype != np.float16 or scales.shape != (out,):
        raise ValueError("scales must be float16 [out]")
    return M, B, g, out, G * g


def codes_to_index(codes: np.ndarray, B: int | None = None) -> np.ndarray:
    """Codeword index of every stored code, as int64.

    A code is the position of the selected codeword inside its codebook
    (MCQ section: the one-hot vector is stored as its index).  uint8 codes are
    their value; int16 codes are their 16-bit pattern read as unsigned.  With
    B given, only the low B bits count (a code of B < 8 or B < 16 bits leaves
    the rest of its bytes unused).
    """
    if codes.dtype == np.uint8 or codes.dtype == np.uint16:
        idx = codes.astype(np.int64)
    elif codes.dtype == np.int16:
        idx = codes.view(np.uint16).astype(np.int64)
    else:
        raise ValueError(f"unsupported code dtype {codes.dtype}")
    return idx if B is None else idx & ((1 << B) - 1)


def decode_fp32(codes, codebooks, scales, rows=None) -> np.ndarray:
    """Dequantized weights in fp32, shape [out][in] (or [len(rows)][in]).

    Figure 2 of the MCQ section: look up one codeword per codebook, sum them
    (fp32, codebook 0 first, m ascending), then multiply by the row's scale.
    """
    M, B, g, out, n_in = _check_layer(codes, codebooks, scales)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        codes = codes[rows]
        scales = scales[rows]
    idx = codes_to_index(codes, B)                   # [r][G][M]
    acc = codebooks[0][idx[:, :, 0]].astype(np.float32)          # [r][G][g]
    for m in range(1, M):
        acc = acc + codebooks[m][idx[:, :, m]].astype(np.float32)
    w = acc * scales.astype(np.float32)[:, None, None]
    return w.reshape(w.shape[0], n_in)


def decode_fp16(codes, codebooks, scales, rows=None) -> np.ndarray:
    """fp16 weights: the fp32 decode rounded to nearest-even (subnormals kept)."""
    return decode_fp32(codes, codebooks, scales, rows).astype(np.float16)


def decode_loop(codes, codebooks, scales) -> np.ndarray:
    """Same decode as ``decode_fp32``, written as explicit loops (tiny layers only).

    Independent second reading of the MCQ-section definition, used to pin the
    vectorised gather.  Each sum and product is rounded to fp32 one operation
    at a time.
    """
    M, B, g, out, n_in = _check_layer(codes, codebooks, scales)
    G = n_in // g
    w = np.zeros((out, n_in), dtype=np.float32)
    f32 = np.float32
    for i in range(out):
        s = f32(scales[i])
        for j in range(G):
            for t in range(g):
                acc = None
                for m in range(M):
                    c = int(codes[i, j, m])
                    if codes.dtype == np.int16 and c < 0:
                        c += 1 << 16
                    c %= 1 << B
                    v = f32(codebooks[m, c, t])
                    acc = v if acc is None else f32(acc + v)
                w[i, j * g + t] = f32(acc * s)
    return w


# ---------------------------------------------------------------------------
# Bit-packed codes
#
# "Key AQLM quantization parameters": a B that is not a multiple of 8 leaves
# unused bits in the bytes that hold each code.  The packed storage drops them.
# Reading (the pages give no packed layout): the codes in their stored order
# ([out][in/g][M] flattened, code n = (i * G + j) * M + m) form one bit stream,
# code n in bits [n * B, n * B + B), least significant bit first; bit b of the
# stream is bit b % 32 of 32-bit word b // 32 (words little-endian), and the
# stream is padded with zero bits to a whole number of words.  Rows are not
# padded, so a row may start inside a word.


def packed_words(n_codes: int, B: int) -> int:
    """Number of 32-bit words that hold n_codes codes of B bits."""
    return (n_codes * B + 31) // 32


def pack_codes(codes: np.ndarray, B: int) -> np.ndarray:
    """The uint32 word stream of the codes' indices (low B bits), code after code, LSB first."""
    idx = codes_to_index(codes, B).reshape(-1)
    bits = ((idx[:, None] >> np.arange(B, dtype=np.int64)[None, :]) & 1).astype(np.uint8).reshape(-1)
    total = packed_words(idx.size, B) * 32
    stream = np.zeros(total, np.uint8)
    stream[:bits.size] = bits
    return np.packbits(stream, bitorder="little").view("<u4").astype(np.uint32)


def unpack_codes(words: np.ndarray, B: int, shape) -> np.ndarray:
    """Indices (int64, shape) of the codes in a packed word stream."""
    n = int(np.prod(shape))
    if words.size < packed_words(n, B):
        raise ValueError("the word stream is shorter than the codes it should hold")
    stream = np.unpackbits(np.ascontiguousarray(words, dtype="<u4").view(np.uint8), bitorder="little")
    bits = stream[:n * B].reshape(n, B).astype(np.int64)
    return (bits << np.arange(B, dtype=np.int64)[None, :]).sum(1).reshape(shape)


def packed_to_stored(words, M, B, g, out, n_in) -> np.ndarray:
    """The whole-byte code array [out][in/g][M] that a packed stream encodes."""
    idx = unpack_codes(words, B, (out, n_in // g, M))
    return idx.astype(np.uint8) if B <= 8 else idx.astype(np.uint16).view(np.int16)


def decode_fp32_packed(words, codebooks, scales, M, B, g, out, n_in, rows=None) -> np.ndarray:
    """decode_fp32 of the layer whose codes are the packed stream `words`."""
    return decode_fp32(packed_to_stored(words, M, B, g, out, n_in), codebooks, scales, rows)


def linear_ref_f64(codes, codebooks, scales, x) -> np.ndarray:
    """y[b][i] = sum_k W[i][k] * x[b][k] in float64, W from ``decode_fp32``.

    The matrix product on dequantized weights that Figure 2 of the MCQ
    section feeds; x is [T][in] fp16, the result [T][out] float64.
    """
    w = decode_fp32(codes, codebooks, scales)
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T][in]")
    return (w.astype(np.float64) @ x.astype(np.float64).T).T


def linear_ref_rows_f64(codes, codebooks, scales, x, rows) -> np.ndarray:
    """Columns ``rows`` of the reference output: y[:, rows], float64 [T][len(rows)].

    For full-size layers where decoding all of W on the host would be slow.
    """
    w = decode_fp32(codes, codebooks, scales, rows=rows)
    return (w.astype(np.float64) @ np.asarray(x).astype(np.float64).T).T


def bits_per_weight_terms(M, B, g, d_out, d_in):
    """Average bits per parameter of one weight matrix, split by stored item.

    "Memory footprint of AQLM-quantized models": codes (M codes of B bits for
    each of d_out*d_in/g groups), codebooks (M * 2^B codewords of g fp16
    values) and scales (d_out fp16 values), each divided by d_out*d_in.
    """
    n = d_out * d_in
    codes = M * B * (d_out * d_in // g) / n
    codebooks = M * (2 ** B) * g * 16 / n
    scales = d_out * 16 / n
    return {"codes": codes, "codebooks": codebooks, "scales": scales,
            "total": codes + codebooks + scales}


def bits_per_weight(M, B, g, d_out, d_in) -> float:
    return bits_per_weight_terms(M, B, g, d_out, d_in)["total"]


def parity_errors(y, y_ref):
    """(relative L2 error, max abs error, max |y_ref|) in float64 over all outputs."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    diff = y - y_ref
    ref_norm = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(diff)) / ref_norm if ref_norm > 0 else float(np.linalg.norm(diff))
    return rel, float(np.max(np.abs(diff))) if diff.size else 0.0, float(np.max(np.abs(y_ref))) if y_ref.size else 0.0


# GEMV/GEMM acceptance: relative L2 <= 1e-3 and max abs <= 1e-2 * max|y_ref|.
REL_L2_TOL = 1e-3
MAX_ABS_FRAC = 1e-2


def within_tolerance(y, y_ref):
    rel, mx, ref_max = parity_errors(y, y_ref)
    return rel <= REL_L2_TOL and mx <= MAX_ABS_FRAC * ref_max


# ---------------------------------------------------------------------------
# Encoding with fixed codebooks, and residual k-means codebook initialisation
#
# "The AQLM Quantization Algorithm, Explained", section "The AQLM quantization
# procedure": per linear layer, the codes are learned first with the codebooks
# fixed, and those codebooks are initialised with a residual k-means approach.
# The learning loss itself did not survive text extraction and is weighted by
# calibration activations, so these are the data-free readings:
#
# * a group's target is its weights divided by the row's scale (scales are
#   given; the pages do not say how they are initialised), in fp32;
# * codes are chosen greedily, codebook 0 first: the code for codebook m is the
#   nearest codeword (squared Euclidean distance) to what the earlier
#   codebooks left over, and that codeword is subtracted;
# * residual k-means runs Lloyd's algorithm on those leftovers for codebook 0,
#   then on what codebook 0 leaves for codebook 1, and so on; its seeds are
#   given groups (random numbers the method draws are inputs);
# * distances are sum_t (r_t - c_t)^2 in fp32, t ascending, each operation
#   rounded (no fused multiply-add); ties go to the lowest index;
# * a centroid is the mean of its members, accumulated exactly in fixed point
#   (each coordinate rounded to a multiple of 2^-24, summed as integers) and
#   divided in float64, then rounded to fp32; an empty cluster keeps its
#   centroid; the codebook is the fp16 rounding of the final centroids, and the
#   codes are assigned against that fp16 codebook.

KMEANS_FIXED_POINT = 2.0 ** 24


def group_targets(w, scales, g):
    """[out*in/g][g] fp32 group vectors: W[i][j*g+t] / s_i, one fp32 division each."""
    w = np.asarray(w)
    if w.dtype != np.float16 or scales.dtype != np.float16:
        raise ValueError("w and scales must be float16")
    out, n_in = w.shape
    if n_in % g or scales.shape != (out,):
        raise ValueError("w must be [out][in] with in % g == 0, scales [out]")
    r = w.astype(np.float32) / scales.astype(np.float32)[:, None]
    return r.reshape(out * (n_in // g), g)


def nearest_codeword(r, cb32, chunk=1024):
    """Index of the nearest row of cb32 [K][g] (fp32) for every row of r [N][g].

    Distance sum_t (r_t - c_t)^2 in fp32, t ascending; the lowest index wins a tie.
    """
    N, g = r.shape
    K = cb32.shape[0]
    best = np.zeros(N, np.int64)
    best_d = np.full(N, np.inf, np.float32)
    for k0 in range(0, K, chunk):
        c = cb32[k0:k0 + chunk]
        d = np.zeros((N, c.shape[0]), np.float32)
        for t in range(g):
            e = r[:, None, t] - c[None, :, t]
            d = d + e * e
        kk = np.argmin(d, axis=1)
        dd = d[np.arange(N), kk]
        upd = dd < best_d
        best[upd] = kk[upd] + k0
        best_d[upd] = dd[upd]
    return best


def _store_codes(idx, B):
    return idx.astype(np.uint8) if B <= 8 else idx.astype(np.uint16).view(np.int16)


def encode_greedy(w, scales, codebooks):
    """Codes [out][in/g][M] for W with fixed codebooks (greedy residual, m ascending)."""
    M, K, g = codebooks.shape
    B = K.bit_length() - 1
    r = group_targets(w, scales, g).copy()
    idx = np.zeros((r.shape[0], M), np.int64)
    for m in range(M):
        cb = codebooks[m].astype(np.float32)
        idx[:, m] = nearest_codeword(r, cb)
        r = r - cb[idx[:, m]]
    out = w.shape[0]
    return _store_codes(idx.reshape(out, -1, M), B)


def kmeans_centroids(r, labels, prev):
    """Lloyd update: per cluster, the fixed-point mean of its members (empty: previous centroid)."""
    K, g = prev.shape
    q = np.rint(r.astype(np.float64) * KMEANS_FIXED_POINT).astype(np.int64)
    sums = np.zeros((K, g), np.int64)
    np.add.at(sums, labels, q)
    counts = np.bincount(labels, minlength=K).astype(np.int64)
    c = prev.copy()
    nz = counts > 0
    c[nz] = (sums[nz].astype(np.float64) / KMEANS_FIXED_POINT / counts[nz, None].astype(np.float64)).astype(np.float32)
    return c


def kmeans_residual_init(w, scales, init_groups, M, B, g, iters):
    """Residual k-means: (codebooks [M][2^B][g] fp16, codes [out][in/g][M]).

    init_groups [M][2^B]: the group indices whose leftovers seed each codebook.
    """
    K = 1 << B
    init_groups = np.asarray(init_groups, np.int64)
    if init_groups.shape != (M, K):
        raise ValueError("init_groups must be [M][2^B]")
    r = group_targets(w, scales, g).copy()
    codebooks = np.zeros((M, K, g), np.float16)
    idx = np.zeros((r.shape[0], M), np.int64)
    for m in range(M):
        c = r[init_groups[m]].copy()
        for _ in range(iters):
            c = kmeans_centroids(r, nearest_codeword(r, c), c)
        codebooks[m] = c.astype(np.float16)
        cb = codebooks[m].astype(np.float32)
        idx[:, m] = nearest_codeword(r, cb)
        r = r - cb[idx[:, m]]
    return codebooks, _store_codes(idx.reshape(w.shape[0], -1, M), B)


def kmeans_objective(r, cb32, labels):
    """Sum of squared distances of r to their centroids (float64)."""
    d = r.astype(np.float64) - cb32.astype(np.float64)[labels]
    return float((d * d).sum())
