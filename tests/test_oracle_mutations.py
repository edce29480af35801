"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle.py catch every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "drop_second_codebook": (
        "for m in range(1, M):\n        acc = acc + codebooks[m][idx[:, :, m]].astype(np.float32)", "pass"),
    "int16_codes_signed": (
        "idx = codes.view(np.uint16).astype(np.int64)", "idx = codes.astype(np.int64)"),
    "sum_starts_at_plus_zero": (
        "acc = codebooks[0][idx[:, :, 0]].astype(np.float32)          # [r][G][g]\n    for m in range(1, M):",
        "acc = np.zeros(idx.shape[:2] + (g,), np.float32)\n    for m in range(0, M):"),
    "scale_off_by_rounding": (
        "w = acc * scales.astype(np.float32)[:, None, None]",
        "w = acc * (scales.astype(np.float32)[:, None, None] * np.float32(1.0001))"),
    "codes_m_swapped": (
        "acc = codebooks[0][idx[:, :, 0]]", "acc = codebooks[0][idx[:, :, M - 1]]"),
    "column_order_t_major": (
        "return w.reshape(w.shape[0], n_in)", "return w.transpose(0, 2, 1).reshape(w.shape[0], n_in)"),
    "product_transposed": (
        "return (w.astype(np.float64) @ x.astype(np.float64).T).T",
        "return (w.astype(np.float64) @ x.astype(np.float64).T)"),
    "fp16_running_sum": (
        "acc = acc + codebooks[m][idx[:, :, m]].astype(np.float32)",
        "acc = (acc.astype(np.float16) + codebooks[m][idx[:, :, m]]).astype(np.float32)"),
    "bpw_scale_32bit": ("scales = d_out * 16 / n", "scales = d_out * 32 / n"),
    "index_ignores_b_bits": (
        "return idx if B is None else idx & ((1 << B) - 1)", "return idx"),
    "loop_ignores_b_bits": ("                    c %= 1 << B\n", ""),
    "codebook_m_reversed": (
        "acc = acc + codebooks[m][idx[:, :, m]].astype(np.float32)",
        "acc = acc + codebooks[M - m][idx[:, :, m]].astype(np.float32)"),
    "bpw_one_codebook": ("codebooks = M * (2 ** B) * g * 16 / n", "codebooks = (2 ** B) * g * 16 / n"),
}


# Mistakes in the encoder and residual k-means, caught by test_oracle_encode.py.
ENCODE_MUTANTS = {
    "greedy_no_subtract": ("        r = r - cb[idx[:, m]]\n    out = w.shape[0]", "    out = w.shape[0]"),
    "ties_take_last": ("kk = np.argmin(d, axis=1)", "kk = d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)"),
    "distance_abs": ("d = d + e * e", "d = d + np.abs(e)"),
    "centroid_is_a_sum": (
        " / KMEANS_FIXED_POINT / counts[nz, None].astype(np.float64)).astype(np.float32)",
        " / KMEANS_FIXED_POINT).astype(np.float32)"),
    "kmeans_residual_not_chained": ("        r = r - cb[idx[:, m]]\n    return codebooks", "    return codebooks"),
    "chunk_ties_take_later": ("upd = dd < best_d", "upd = dd <= best_d"),
    "centroid_plain_float_mean": (
        "q = np.rint(r.astype(np.float64) * KMEANS_FIXED_POINT).astype(np.int64)\n    sums = np.zeros((K, g), np.int64)",
        "q = r.astype(np.float64) * KMEANS_FIXED_POINT\n    sums = np.zeros((K, g), np.float64)"),
    "centroid_rounds_down": ("q = np.rint(r.astype", "q = np.floor(r.astype"),
    "centroid_finer_grid": ("KMEANS_FIXED_POINT = 2.0 ** 24", "KMEANS_FIXED_POINT = 2.0 ** 30"),
    "targets_times_scale": ("r = w.astype(np.float32) / scales.astype(np.float32)[:, None]",
                            "r = w.astype(np.float32) * scales.astype(np.float32)[:, None]"),
}
# Mistakes in the bit-packed codes, caught by test_oracle_packed.py.
PACKED_MUTANTS = {
    "pack_msb_first": ("bits = ((idx[:, None] >> np.arange(B, dtype=np.int64)[None, :]) & 1)",
                       "bits = ((idx[:, None] >> np.arange(B - 1, -1, -1, dtype=np.int64)[None, :]) & 1)"),
    "pack_big_endian_bits": ('return np.packbits(stream, bitorder="little")', 'return np.packbits(stream, bitorder="big")'),
    "pack_codebook_major": ("idx = codes_to_index(codes, B).reshape(-1)",
                            "idx = np.moveaxis(codes_to_index(codes, B), -1, 0).reshape(-1)"),
    "pack_one_bit_short": ("total = packed_words(idx.size, B) * 32", "total = packed_words(idx.size, B - 1) * 32"),
}
CASES = [(n, MUTANTS[n], "test_oracle.py") for n in sorted(MUTANTS)] + \
        [(n, ENCODE_MUTANTS[n], "test_oracle_encode.py") for n in sorted(ENCODE_MUTANTS)] + \
        [(n, PACKED_MUTANTS[n], "test_oracle_packed.py") for n in sorted(PACKED_MUTANTS)]


@pytest.mark.parametrize("name,mutant,pins", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_mutant(name, mutant, pins, tmp_path):
    before, after = mutant
    src = open(os.path.join(ROOT, "oracle", "aqlm_oracle.py")).read()
    assert before in src, f"mutation site for {name} not found"
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst, ignore=shutil.ignore_patterns("__pycache__"))
    (dst / "aqlm_oracle.py").write_text(src.replace(before, after))
    env = dict(os.environ, AQLM_ORACLE_MUTANT_DIR=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived:\n{r.stdout[-2000:]}"
