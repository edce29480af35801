"""AQLM 2-bit quantized linear layer for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libaqlm.so``, declared in ``include/aqlm.h``); this package holds the thin
ctypes binding to it and the seeded synthetic-input generators.
"""
