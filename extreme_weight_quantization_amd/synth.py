"""Seeded synthetic inputs for AQLM quantized linear layers.

Draws only random numbers: codebooks, codes, scales and activations with the
shapes and distributions of the Llama-2-7B/70B projection layers.  It holds
none of the method's arithmetic, so the HIP library's tests and the CPU
oracle can both take their inputs from here.

Recipe (numpy ``default_rng(seed)``, PCG64), drawn in this order:
codebooks ~ N(0, sigma) as float64 rounded to fp16, codes uniform over every
B-bit pattern, scales ~ U(0.5, 1.5) rounded to fp16, activations ~ N(0, 1)
rounded to fp16.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Scheme name -> (M codebooks, B bits per code, g group size, codebook sigma).
SCHEMES = {
    "2x8": (2, 8, 8, 0.05),
    "1x16": (1, 16, 8, 0.02),
}

# Llama-2 projection shapes (out, in).
LLAMA2_7B_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))
LLAMA2_70B_SHAPES = ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672))
# One 7B decoder block's projections: q, k, v, o, gate, up, down.
LLAMA2_7B_BLOCK = ((4096, 4096),) * 4 + ((11008, 4096),) * 2 + ((4096, 11008),)


@dataclass
class Layer:
    scheme: str
    M: int
    B: int
    g: int
    codebooks: np.ndarray   # fp16 [M][2^B][g]
    codes: np.ndarray       # uint8 (B=8) or int16 (B=16) [out][in/g][M]
    scales: np.ndarray      # fp16 [out]
    x: np.ndarray           # fp16 [T][in]

    @property
    def out_features(self):
        return self.codes.shape[0]

    @property
    def in_features(self):
        return self.codes.shape[1] * self.g


def scheme_name(M: int, B: int, g: int) -> str:
    return f"{M}x{B}g{g}"


def make_layer(scheme: str, out: int, n_in: int, batch: int = 1, seed: int = 0,
               sigma: float | None = None) -> Layer:
    """One synthetic quantized layer plus activations, seeded (a named scheme)."""
    M, B, g, default_sigma = SCHEMES[scheme]
    layer = make_layer_mbg(M, B, g, out, n_in, batch, seed, default_sigma if sigma is None else sigma)
    layer.scheme = scheme
    return layer


def make_layer_mbg(M: int, B: int, g: int, out: int, n_in: int, batch: int = 1, seed: int = 0,
                   sigma: float = 0.05) -> Layer:
    """One synthetic layer of any scheme: M codebooks of 2^B codewords of g entries.

    Codes are stored in whole bytes (uint8 for B <= 8, int16 bit patterns for
    9 <= B <= 16) and drawn uniform over the 2^B valid indices.
    """
    if n_in % g:
        raise ValueError("in must be a multiple of g")
    if not (1 <= B <= 16 and M >= 1 and g >= 1):
        raise ValueError("need M >= 1, 1 <= B <= 16, g >= 1")
    rng = np.random.default_rng(seed)
    codebooks = rng.normal(0.0, sigma, size=(M, 1 << B, g)).astype(np.float16)
    if B <= 8:
        codes = rng.integers(0, 1 << B, size=(out, n_in // g, M), dtype=np.uint8)
    else:
        codes = rng.integers(0, 1 << B, size=(out, n_in // g, M), dtype=np.uint16).view(np.int16)
    scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
    x = rng.normal(0.0, 1.0, size=(batch, n_in)).astype(np.float16)
    return Layer(scheme_name(M, B, g), M, B, g, codebooks, codes, scales, x)


def make_activations(n_in: int, batch: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, 1.0, size=(batch, n_in)).astype(np.float16)


def adversarial_codebooks(scheme: str, seed: int = 0) -> np.ndarray:
    """Codebooks holding signed zeros, fp16 subnormals and the largest magnitudes.

    Entries 0 and 2^B-1 (the extreme codes) get the special values so that
    extreme codes select them.
    """
    M, B, g, sigma = SCHEMES[scheme]
    rng = np.random.default_rng(seed)
    cb = rng.normal(0.0, sigma, size=(M, 1 << B, g)).astype(np.float16)
    sub = np.array([2.0 ** -24, -(2.0 ** -24), 2.0 ** -20, -(2.0 ** -15) * 1.5,
                    6.0e-5, -3.0e-6, 2.0 ** -14 * 0.999, -(2.0 ** -17)], dtype=np.float16)
    zeros = np.array([0.0, -0.0, 0.0, -0.0, -0.0, 0.0, -0.0, -0.0], dtype=np.float16)
    big = np.array([1024.0, -1024.0, 2047.0, -2048.0, 512.5, -999.0, 1500.0, -1.0], dtype=np.float16)
    for m in range(M):
        cb[m, 0, :] = zeros
        cb[m, (1 << B) - 1, :] = sub
        cb[m, 1, :] = big
        cb[m, 2, :] = -zeros
        # a band of subnormal-sized entries
        cb[m, 3:64, :] = (rng.normal(0.0, 2.0 ** -18, size=(61, g))).astype(np.float16)
    return cb
