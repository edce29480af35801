"""AQLM 2-bit quantized linear layer for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libaqlm.so``, declared in ``include/aqlm.h``).  ``binding`` is the thin
ctypes layer over it; ``synth`` draws seeded synthetic layers.  The library
is loaded on first use and its absence is an error: there is no fallback.
"""
from .binding import (  # noqa: F401
    AqlmError,
    SliceLists,
    aqlm_linear_gemv_lists,
    aqlm_linear_gemv_lists_fused,
    aqlm_linear_gemv_lists_noalloc,
    aqlm_pack_codes,
    aqlm_linear_gemv_packed,
    aqlm_linear_gemm_packed,
    aqlm_linear_decode_packed,
    packed_codes_bytes,
    aqlm_lists_pack,
    aqlm_linear_decode,
    aqlm_linear_gemm,
    aqlm_linear_gemm_dequant,
    gemm_dequant_workspace_bytes,
    aqlm_linear_gemv,
    aqlm_linear_gemv_fused,
    aqlm_encode_greedy,
    aqlm_kmeans_init,
    kmeans_workspace_bytes,
    lists_fused_workspace_bytes,
    lists_table_bytes,
    lists_workspace_bytes,
    load_library,
    status_str,
)
