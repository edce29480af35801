"""ctypes binding of libaqlm.so (declared in include/aqlm.h).

Argument marshalling only: tensors are checked for device, dtype and
contiguity, their data pointers and sizes are handed to the C ABI together
with torch's current HIP stream, and status codes become exceptions.  Every
step of the computation runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaqlm.so")

AQLM_OK, AQLM_ERR_NULL, AQLM_ERR_SHAPE, AQLM_ERR_SCHEME, AQLM_ERR_ALIGN, AQLM_ERR_HIP, AQLM_ERR_SCRATCH = range(7)
EXPORTED = ("aqlm_linear_gemv", "aqlm_linear_gemv_fused", "aqlm_linear_gemm", "aqlm_linear_decode",
            "aqlm_encode_greedy", "aqlm_kmeans_workspace_bytes", "aqlm_kmeans_init",
            "aqlm_lists_table_bytes", "aqlm_lists_workspace_bytes", "aqlm_lists_plan", "aqlm_lists_fill",
            "aqlm_linear_gemv_lists", "aqlm_linear_gemv_lists_fused", "aqlm_lists_fused_workspace_bytes",
            "aqlm_linear_gemm_dequant", "aqlm_gemm_dequant_workspace_bytes", "aqlm_linear_gemv_lists_noalloc",
            "aqlm_packed_codes_bytes", "aqlm_pack_codes", "aqlm_linear_gemv_packed", "aqlm_linear_gemm_packed",
            "aqlm_linear_decode_packed",
            "aqlm_status_str", "aqlm_last_hip_error", "aqlm_version")
FUSED_MAX_LAYERS = 8   # AQLM_FUSED_MAX_LAYERS

_lib = None
_lock = threading.Lock()


class AqlmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libaqlm.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m extreme_weight_quantization_amd.build`")
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        for name in ("aqlm_linear_gemv", "aqlm_linear_gemm", "aqlm_linear_decode", "aqlm_linear_gemv_packed",
                     "aqlm_linear_gemm_packed", "aqlm_linear_decode_packed"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, i64, i64, i64, vp]
            fn.restype = ci
        pp = ctypes.POINTER(vp)
        lib.aqlm_linear_gemv_fused.argtypes = [ci, pp, pp, pp, ctypes.POINTER(i64), vp, pp,
                                               ci, ci, ci, i64, i64, vp]
        lib.aqlm_linear_gemv_fused.restype = ci
        lib.aqlm_encode_greedy.argtypes = [vp, vp, vp, vp, ci, ci, ci, i64, i64, vp]
        lib.aqlm_encode_greedy.restype = ci
        lib.aqlm_kmeans_workspace_bytes.argtypes = [ci, ci, ci, ctypes.POINTER(i64)]
        lib.aqlm_kmeans_workspace_bytes.restype = ci
        lib.aqlm_kmeans_init.argtypes = [vp, vp, vp, vp, vp, vp, i64, ci, ci, ci, i64, i64, ci, vp]
        lib.aqlm_kmeans_init.restype = ci
        for name in ("aqlm_lists_table_bytes", "aqlm_lists_workspace_bytes"):
            getattr(lib, name).argtypes = [ci, ci, ci, i64, i64, ctypes.POINTER(i64)]
            getattr(lib, name).restype = ci
        lib.aqlm_lists_plan.argtypes = [vp, vp, ci, ci, ci, i64, i64, vp]
        lib.aqlm_lists_plan.restype = ci
        lib.aqlm_lists_fill.argtypes = [vp, vp, vp, i64, ci, ci, ci, i64, i64, vp]
        lib.aqlm_lists_fill.restype = ci
        lib.aqlm_linear_gemv_lists.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, i64, ci, ci, ci, i64, i64, i64, vp]
        lib.aqlm_linear_gemv_lists.restype = ci
        lib.aqlm_linear_gemv_lists_noalloc.argtypes = [vp, vp, i64, vp, vp, vp, vp, ci, ci, ci, i64, i64, i64, vp]
        lib.aqlm_linear_gemv_lists_noalloc.restype = ci
        lib.aqlm_linear_gemv_lists_fused.argtypes = [ci, pp, pp, ctypes.POINTER(i64), pp, pp, ctypes.POINTER(i64),
                                                     vp, pp, vp, i64, ci, ci, ci, i64, i64, vp]
        lib.aqlm_linear_gemv_lists_fused.restype = ci
        lib.aqlm_lists_fused_workspace_bytes.argtypes = [ci, ctypes.POINTER(i64), ci, ci, ci, i64,
                                                         ctypes.POINTER(i64)]
        lib.aqlm_lists_fused_workspace_bytes.restype = ci
        lib.aqlm_linear_gemm_dequant.argtypes = [vp, vp, vp, vp, vp, vp, i64, ci, ci, ci, i64, i64, i64, vp]
        lib.aqlm_linear_gemm_dequant.restype = ci
        lib.aqlm_gemm_dequant_workspace_bytes.argtypes = [ci, ci, ci, i64, i64, ctypes.POINTER(i64)]
        lib.aqlm_gemm_dequant_workspace_bytes.restype = ci
        lib.aqlm_packed_codes_bytes.argtypes = [ci, ci, ci, i64, i64, ctypes.POINTER(i64)]
        lib.aqlm_packed_codes_bytes.restype = ci
        lib.aqlm_pack_codes.argtypes = [vp, vp, ci, ci, ci, i64, i64, vp]
        lib.aqlm_pack_codes.restype = ci
        lib.aqlm_status_str.argtypes = [ci]
        lib.aqlm_status_str.restype = ctypes.c_char_p
        lib.aqlm_last_hip_error.argtypes = []
        lib.aqlm_last_hip_error.restype = ci
        lib.aqlm_version.argtypes = []
        lib.aqlm_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def status_str(status: int) -> str:
    return load_library().aqlm_status_str(int(status)).decode()


def _check(status: int):
    if status == AQLM_OK:
        return
    lib = load_library()
    msg = lib.aqlm_status_str(status).decode()
    if status == AQLM_ERR_HIP:
        raise AqlmError(status, f"{msg} (hipError_t {lib.aqlm_last_hip_error()})")
    err = AqlmError(status, msg)
    raise ValueError(msg) from err


def _scheme(codes: torch.Tensor, codebooks: torch.Tensor):
    if codebooks.dim() != 3:
        raise ValueError("codebooks must be [M][2^B][g]")
    M, K, g = codebooks.shape
    B = K.bit_length() - 1
    if K != 1 << B:
        raise ValueError("the codebook size must be a power of two")
    if (B <= 8) != (codes.dtype == torch.uint8):
        raise ValueError("codes must be uint8 for B <= 8 and int16 for 9 <= B <= 16")
    return int(M), int(B), int(g)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _same_device(named):
    """All tensors (name, tensor) on one GPU: the kernels get raw pointers of one device."""
    devs = {(t.device.type, t.device.index) for _, t in named if t is not None}
    if len(devs) > 1:
        raise ValueError("tensors are on different devices: " +
                         ", ".join(f"{n} on {t.device}" for n, t in named if t is not None))


def _check_tensors(codes, codebooks, scales, x):
    """Device, dtype, contiguity and the shapes that tie codes, codebooks and scales together
    (codes [out][in/g][M] with M from the codebooks, scales [out]); a mismatch would make the
    kernels read past a buffer, so it is refused here, before any launch."""
    named = (("codes", codes), ("codebooks", codebooks), ("scales", scales), ("x", x))
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _same_device(named)
    if codebooks.dtype != torch.float16 or scales.dtype != torch.float16:
        raise ValueError("codebooks and scales must be float16")
    if codes.dtype not in (torch.uint8, torch.int16):
        raise ValueError("codes must be uint8 (B=8) or int16 (B=16)")
    if x is not None and x.dtype != torch.float16:
        raise ValueError("x must be float16")
    if codes.dim() != 3:
        raise ValueError("codes must be [out][in/g][M]")
    if codebooks.dim() == 3 and codes.shape[2] != codebooks.shape[0]:
        raise ValueError(f"codes hold {codes.shape[2]} codes per group but there are "
                         f"{codebooks.shape[0]} codebooks")
    if scales.shape != (codes.shape[0],):
        raise ValueError(f"scales must be [{codes.shape[0]}] (one per output row)")


def _linear(fn_name, codes, codebooks, scales, x, y):
    _check_tensors(codes, codebooks, scales, x)
    M, B, g = _scheme(codes, codebooks)
    out, G = int(codes.shape[0]), int(codes.shape[1])
    n_in = G * g
    if x.dim() != 2 or x.shape[1] != n_in:
        raise ValueError(f"x must be [batch][{n_in}]")
    batch = int(x.shape[0])
    if y is None:
        y = torch.empty((batch, out), dtype=torch.float16, device=x.device)
    elif y.shape != (batch, out) or y.dtype != torch.float16 or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous float16 [{batch}][{out}] tensor")
    _same_device((("x", x), ("y", y)))
    fn = getattr(load_library(), fn_name)
    _check(fn(_ptr(codes), _ptr(codebooks), _ptr(scales), _ptr(x), _ptr(y), M, B, g,
              out, n_in, batch, _stream(x.device)))
    return y


def aqlm_linear_gemv(codes, codebooks, scales, x, y=None):
    """y[b] = W x[b] for a decode batch of 1..16 rows of x (see aqlm.h)."""
    return _linear("aqlm_linear_gemv", codes, codebooks, scales, x, y)


def aqlm_linear_gemv_fused(layers, x, ys=None):
    """[y_l] for layers l = (codes, codebooks, scales) that all multiply the same x, in one launch.

    The layers share the scheme and `in`; each has its own rows.  Results equal
    separate aqlm_linear_gemv calls bit for bit (see aqlm.h)."""
    layers = list(layers)
    if not 1 <= len(layers) <= FUSED_MAX_LAYERS:
        raise ValueError(f"1 to {FUSED_MAX_LAYERS} layers per call")
    scheme = None
    outs = []
    for codes, codebooks, scales in layers:
        _check_tensors(codes, codebooks, scales, x)
        sch = _scheme(codes, codebooks)
        if scheme is not None and sch != scheme:
            raise ValueError("all layers of a fused call must use the same (M, B, g)")
        scheme = sch
        outs.append(int(codes.shape[0]))
    M, B, g = scheme
    n_in = int(layers[0][0].shape[1]) * g
    for codes, _, _ in layers:
        if int(codes.shape[1]) * g != n_in:
            raise ValueError("all layers of a fused call must have the same in")
    if x.dim() != 2 or x.shape[1] != n_in:
        raise ValueError(f"x must be [batch][{n_in}]")
    batch = int(x.shape[0])
    if ys is None:
        ys = [torch.empty((batch, o), dtype=torch.float16, device=x.device) for o in outs]
    else:
        ys = list(ys)
        if len(ys) != len(layers):
            raise ValueError("one output per layer")
        for y, o in zip(ys, outs):
            if y.shape != (batch, o) or y.dtype != torch.float16 or not y.is_contiguous():
                raise ValueError(f"y must be a contiguous float16 [{batch}][{o}] tensor")
            _same_device((("x", x), ("y", y)))
    n = len(layers)
    arr = ctypes.c_void_p * n
    c_codes = arr(*[l[0].data_ptr() for l in layers])
    c_cb = arr(*[l[1].data_ptr() for l in layers])
    c_s = arr(*[l[2].data_ptr() for l in layers])
    c_y = arr(*[y.data_ptr() for y in ys])
    c_out = (ctypes.c_int64 * n)(*outs)
    _check(load_library().aqlm_linear_gemv_fused(n, c_codes, c_cb, c_s, c_out, _ptr(x), c_y,
                                                 M, B, g, n_in, batch, _stream(x.device)))
    return ys


def aqlm_linear_gemm(codes, codebooks, scales, x, y=None):
    """Y = X W^T for a prefill batch of tokens (see aqlm.h)."""
    return _linear("aqlm_linear_gemm", codes, codebooks, scales, x, y)


def gemm_dequant_workspace_bytes(M: int, B: int, g: int, out: int, n_in: int) -> int:
    """Bytes of workspace aqlm_linear_gemm_dequant needs (the decoded weights; 0 when in % 64 != 0)."""
    n = ctypes.c_int64(0)
    _check(load_library().aqlm_gemm_dequant_workspace_bytes(M, B, g, out, n_in, ctypes.byref(n)))
    return int(n.value)


def aqlm_linear_gemm_dequant(codes, codebooks, scales, x, y=None, workspace=None):
    """Y = X W^T in two passes: W decoded once into the workspace, then a dense fp16 product (see aqlm.h)."""
    _check_tensors(codes, codebooks, scales, x)
    M, B, g = _scheme(codes, codebooks)
    out, G = int(codes.shape[0]), int(codes.shape[1])
    n_in = G * g
    if x.dim() != 2 or x.shape[1] != n_in:
        raise ValueError(f"x must be [batch][{n_in}]")
    batch = int(x.shape[0])
    if y is None:
        y = torch.empty((batch, out), dtype=torch.float16, device=x.device)
    elif y.shape != (batch, out) or y.dtype != torch.float16 or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous float16 [{batch}][{out}] tensor")
    need = gemm_dequant_workspace_bytes(M, B, g, out, n_in)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    _same_device((("x", x), ("y", y), ("workspace", workspace)))
    _check(load_library().aqlm_linear_gemm_dequant(_ptr(codes), _ptr(codebooks), _ptr(scales), _ptr(x), _ptr(y),
                                                   _ptr(workspace), workspace.numel(), M, B, g, out, n_in, batch,
                                                   _stream(x.device)))
    return y


def aqlm_linear_decode(codes, codebooks, scales, w=None):
    """W16[out][in] = dequantized weights, bit-exact (see aqlm.h)."""
    _check_tensors(codes, codebooks, scales, None)
    M, B, g = _scheme(codes, codebooks)
    out, G = int(codes.shape[0]), int(codes.shape[1])
    if w is None:
        w = torch.empty((out, G * g), dtype=torch.float16, device=codes.device)
    elif w.shape != (out, G * g) or w.dtype != torch.float16 or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous float16 [{out}][{G * g}] tensor")
    _same_device((("codes", codes), ("w", w)))
    _check(load_library().aqlm_linear_decode(_ptr(codes), _ptr(codebooks), _ptr(scales), None,
                                             _ptr(w), M, B, g, out, G * g, 0, _stream(codes.device)))
    return w


# ---------------------------------------------------------------------------
# Bit-packed codes (layout in aqlm.h): an int32 tensor holds the 32-bit words.


def packed_codes_bytes(M: int, B: int, g: int, out: int, n_in: int) -> int:
    """Bytes of the bit-packed codes of a layer [out][n_in] of scheme (M, B, g)."""
    n = ctypes.c_int64(0)
    _check(load_library().aqlm_packed_codes_bytes(M, B, g, out, n_in, ctypes.byref(n)))
    return int(n.value)


def aqlm_pack_codes(codes, B: int, packed=None):
    """The bit-packed stream (int32 words) of whole-byte codes [out][in/g][M] whose indices have B bits."""
    if not (codes.is_cuda and codes.is_contiguous() and codes.dim() == 3):
        raise ValueError("codes must be a contiguous GPU tensor [out][in/g][M]")
    if (B <= 8) != (codes.dtype == torch.uint8) or codes.dtype not in (torch.uint8, torch.int16):
        raise ValueError("codes must be uint8 for B <= 8 and int16 for 9 <= B <= 16")
    out, G, M = (int(v) for v in codes.shape)
    n_words = packed_codes_bytes(M, B, 1, out, G) // 4   # g = 1 with in = G: the same code count
    if packed is None:
        packed = torch.empty((max(n_words, 1),), dtype=torch.int32, device=codes.device)
    elif packed.dtype != torch.int32 or not packed.is_contiguous() or packed.numel() < n_words:
        raise ValueError(f"packed must be a contiguous int32 tensor of at least {n_words} words")
    _same_device((("codes", codes), ("packed", packed)))
    _check(load_library().aqlm_pack_codes(_ptr(codes), _ptr(packed), M, B, 1, out, G, _stream(codes.device)))
    return packed


def _packed_args(packed, codebooks, scales, n_in, x=None):
    for name, t in (("packed", packed), ("codebooks", codebooks), ("scales", scales), ("x", x)):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _same_device((("packed", packed), ("codebooks", codebooks), ("scales", scales), ("x", x)))
    if packed.dtype != torch.int32:
        raise ValueError("packed codes must be an int32 tensor of 32-bit words")
    if codebooks.dtype != torch.float16 or scales.dtype != torch.float16 or codebooks.dim() != 3 or scales.dim() != 1:
        raise ValueError("codebooks [M][2^B][g] and scales [out] must be float16")
    M, K, g = (int(v) for v in codebooks.shape)
    B = K.bit_length() - 1
    if K != 1 << B:
        raise ValueError("the codebook size must be a power of two")
    out = int(scales.shape[0])
    if n_in % g:
        raise ValueError("in must be a multiple of g")
    need = packed_codes_bytes(M, B, g, out, n_in)
    if packed.numel() * 4 < need:
        raise ValueError(f"packed holds {packed.numel() * 4} bytes, the layer needs {need}")
    return M, B, g, out


def _packed_linear(fn_name, packed, codebooks, scales, x, y):
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be float16 [batch][in]")
    n_in, batch = int(x.shape[1]), int(x.shape[0])
    M, B, g, out = _packed_args(packed, codebooks, scales, n_in, x)
    if y is None:
        y = torch.empty((batch, out), dtype=torch.float16, device=x.device)
    elif y.shape != (batch, out) or y.dtype != torch.float16 or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous float16 [{batch}][{out}] tensor")
    _same_device((("x", x), ("y", y)))
    _check(getattr(load_library(), fn_name)(_ptr(packed), _ptr(codebooks), _ptr(scales), _ptr(x), _ptr(y), M, B, g,
                                            out, n_in, batch, _stream(x.device)))
    return y


def aqlm_linear_gemv_packed(packed, codebooks, scales, x, y=None):
    """y = W x at batch 1..16 with W's codes bit-packed (out = scales.shape[0], in = x.shape[1])."""
    return _packed_linear("aqlm_linear_gemv_packed", packed, codebooks, scales, x, y)


def aqlm_linear_gemm_packed(packed, codebooks, scales, x, y=None):
    """Y = X W^T for any batch of tokens, W's codes bit-packed."""
    return _packed_linear("aqlm_linear_gemm_packed", packed, codebooks, scales, x, y)


def aqlm_linear_decode_packed(packed, codebooks, scales, n_in, w=None):
    """W16[out][n_in] from bit-packed codes, bit-exact."""
    M, B, g, out = _packed_args(packed, codebooks, scales, int(n_in))
    if w is None:
        w = torch.empty((out, int(n_in)), dtype=torch.float16, device=packed.device)
    elif w.shape != (out, int(n_in)) or w.dtype != torch.float16 or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous float16 [{out}][{n_in}] tensor")
    _same_device((("packed", packed), ("w", w)))
    _check(load_library().aqlm_linear_decode_packed(_ptr(packed), _ptr(codebooks), _ptr(scales), None, _ptr(w), M, B,
                                                    g, out, int(n_in), 0, _stream(packed.device)))
    return w


def _check_weights(w, scales, g):
    for name, t in (("w", w), ("scales", scales)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    if w.dim() != 2 or scales.shape != (w.shape[0],):
        raise ValueError("w must be [out][in] and scales [out]")
    if w.shape[1] % g:
        raise ValueError("in must be a multiple of g")


def _codes_out(codes, out, G, M, B, device):
    dtype = torch.uint8 if B <= 8 else torch.int16
    if codes is None:
        return torch.empty((out, G, M), dtype=dtype, device=device)
    if codes.shape != (out, G, M) or codes.dtype != dtype or not codes.is_contiguous():
        raise ValueError(f"codes must be a contiguous {dtype} [{out}][{G}][{M}] tensor")
    return codes


def aqlm_encode_greedy(w, scales, codebooks, codes=None):
    """Greedy residual codes [out][in/g][M] of w with fixed codebooks (see aqlm.h)."""
    if codebooks.dim() != 3 or codebooks.dtype != torch.float16 or not codebooks.is_cuda:
        raise ValueError("codebooks must be a float16 GPU tensor [M][2^B][g]")
    M, K, g = (int(v) for v in codebooks.shape)
    B = K.bit_length() - 1
    if K != 1 << B:
        raise ValueError("the codebook size must be a power of two")
    _check_weights(w, scales, g)
    out, n_in = int(w.shape[0]), int(w.shape[1])
    codes = _codes_out(codes, out, n_in // g, M, B, w.device)
    _same_device((("w", w), ("scales", scales), ("codebooks", codebooks), ("codes", codes)))
    _check(load_library().aqlm_encode_greedy(_ptr(w), _ptr(scales), _ptr(codebooks.contiguous()), _ptr(codes),
                                             M, B, g, out, n_in, _stream(w.device)))
    return codes


def kmeans_workspace_bytes(M, B, g) -> int:
    n = ctypes.c_int64(0)
    _check(load_library().aqlm_kmeans_workspace_bytes(M, B, g, ctypes.byref(n)))
    return int(n.value)


def aqlm_kmeans_init(w, scales, seeds, B, g, iters, codebooks=None, codes=None, workspace=None):
    """Residual k-means codebooks [M][2^B][g] and their greedy codes (see aqlm.h).

    seeds: int64 GPU tensor [M][2^B] of group indices (row * in/g + j)."""
    if seeds.dim() != 2 or seeds.dtype != torch.int64 or not seeds.is_cuda or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous int64 GPU tensor [M][2^B]")
    M = int(seeds.shape[0])
    if int(seeds.shape[1]) != 1 << B:
        raise ValueError("seeds must have 2^B columns")
    _check_weights(w, scales, g)
    out, n_in = int(w.shape[0]), int(w.shape[1])
    if codebooks is None:
        codebooks = torch.empty((M, 1 << B, g), dtype=torch.float16, device=w.device)
    elif codebooks.shape != (M, 1 << B, g) or codebooks.dtype != torch.float16 or not codebooks.is_contiguous():
        raise ValueError("codebooks must be a contiguous float16 [M][2^B][g] tensor")
    codes = _codes_out(codes, out, n_in // g, M, B, w.device)
    need = kmeans_workspace_bytes(M, B, g)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    _same_device((("w", w), ("scales", scales), ("seeds", seeds), ("codebooks", codebooks), ("codes", codes),
                  ("workspace", workspace)))
    _check(load_library().aqlm_kmeans_init(_ptr(w), _ptr(scales), _ptr(seeds), _ptr(codebooks), _ptr(codes),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           M, B, g, out, n_in, int(iters), _stream(w.device)))
    return codebooks, codes


def _lists_bytes(fn_name, out, n_in) -> int:
    n = ctypes.c_int64(0)
    _check(getattr(load_library(), fn_name)(1, 16, 8, int(out), int(n_in), ctypes.byref(n)))
    return int(n.value)


def lists_table_bytes(out, n_in) -> int:
    """Bytes of the slice-list table of a 1x16 layer [out][n_in] (see aqlm.h)."""
    return _lists_bytes("aqlm_lists_table_bytes", out, n_in)


def lists_workspace_bytes(out, n_in) -> int:
    """Bytes of workspace aqlm_linear_gemv_lists needs for a 1x16 layer [out][n_in]."""
    return _lists_bytes("aqlm_lists_workspace_bytes", out, n_in)


@dataclass
class SliceLists:
    """The codes of one 1x16 layer regrouped by codebook slice (layout in aqlm.h).

    table and entries are uint8 GPU tensors holding the library's table and
    entries; out and n_in are the layer's shape."""
    table: torch.Tensor
    entries: torch.Tensor
    out: int
    n_in: int

    @property
    def steps(self) -> int:
        return self.entries.numel() // 256


def aqlm_lists_pack(codes) -> SliceLists:
    """Slice lists of 1x16 codes [out][in/8][1] (int16): plan, read the size, allocate, fill.

    Synchronises the current stream once (to read the number of entries)."""
    if not (codes.is_cuda and codes.is_contiguous() and codes.dtype == torch.int16 and codes.dim() == 3
            and codes.shape[2] == 1):
        raise ValueError("codes must be a contiguous int16 GPU tensor [out][in/8][1]")
    out, n_in = int(codes.shape[0]), int(codes.shape[1]) * 8
    lib = load_library()
    table = torch.empty(lists_table_bytes(out, n_in), dtype=torch.uint8, device=codes.device)
    stream = _stream(codes.device)
    _check(lib.aqlm_lists_plan(_ptr(codes), _ptr(table), 1, 16, 8, out, n_in, stream))
    torch.cuda.current_stream(codes.device).synchronize()
    steps = int(table[-8:].cpu().view(torch.int64).item())
    entries = torch.empty(steps * 256, dtype=torch.uint8, device=codes.device)
    _check(lib.aqlm_lists_fill(_ptr(codes), _ptr(table), _ptr(entries), entries.numel(), 1, 16, 8, out, n_in,
                               stream))
    return SliceLists(table, entries, out, n_in)


def aqlm_linear_gemv_lists(lists: SliceLists, codebooks, scales, x, y=None, workspace=None):
    """y = W x at batch 1 over slice lists (see aqlm.h); x is [1][in] (or [0][in])."""
    for name, t in (("codebooks", codebooks), ("scales", scales), ("x", x)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    if codebooks.shape != (1, 1 << 16, 8):
        raise ValueError("codebooks must be [1][65536][8]")
    if x.dim() != 2 or x.shape[1] != lists.n_in or x.shape[0] > 1:
        raise ValueError(f"x must be [1][{lists.n_in}]")
    if scales.shape != (lists.out,):
        raise ValueError(f"scales must be [{lists.out}] (one per output row)")
    batch = int(x.shape[0])
    if y is None:
        y = torch.empty((batch, lists.out), dtype=torch.float16, device=x.device)
    elif y.shape != (batch, lists.out) or y.dtype != torch.float16 or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous float16 [{batch}][{lists.out}] tensor")
    if workspace is None:
        workspace = torch.empty(lists_workspace_bytes(lists.out, lists.n_in), dtype=torch.uint8, device=x.device)
    _same_device((("table", lists.table), ("entries", lists.entries), ("codebooks", codebooks), ("scales", scales),
                  ("x", x), ("y", y), ("workspace", workspace)))
    _check(load_library().aqlm_linear_gemv_lists(
        _ptr(lists.table), _ptr(lists.entries), lists.entries.numel(), _ptr(codebooks), _ptr(scales), _ptr(x),
        _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(), 1, 16, 8, lists.out, lists.n_in,
        batch, _stream(x.device)))
    return y


NOALLOC_SCRATCH_BYTES = 4 << 20   # AQLM_LISTS_NOALLOC_SCRATCH_BYTES


def aqlm_linear_gemv_lists_noalloc(lists: SliceLists, codebooks, scales, x, y):
    """aqlm_linear_gemv_lists with the partial sums in the library's static scratch (see aqlm.h).

    y must be given: the call allocates nothing.  Calls that overlap on one GPU race."""
    for name, t in (("codebooks", codebooks), ("scales", scales), ("x", x), ("y", y)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    if codebooks.shape != (1, 1 << 16, 8):
        raise ValueError("codebooks must be [1][65536][8]")
    if x.dim() != 2 or x.shape[1] != lists.n_in or x.shape[0] > 1:
        raise ValueError(f"x must be [1][{lists.n_in}]")
    if scales.shape != (lists.out,):
        raise ValueError(f"scales must be [{lists.out}] (one per output row)")
    if y.shape != (x.shape[0], lists.out):
        raise ValueError(f"y must be [{x.shape[0]}][{lists.out}]")
    _same_device((("table", lists.table), ("entries", lists.entries), ("codebooks", codebooks), ("scales", scales),
                  ("x", x), ("y", y)))
    _check(load_library().aqlm_linear_gemv_lists_noalloc(
        _ptr(lists.table), _ptr(lists.entries), lists.entries.numel(), _ptr(codebooks), _ptr(scales), _ptr(x),
        _ptr(y), 1, 16, 8, lists.out, lists.n_in, int(x.shape[0]), _stream(x.device)))
    return y


def lists_fused_workspace_bytes(outs, n_in) -> int:
    """Bytes of workspace aqlm_linear_gemv_lists_fused needs for 1x16 layers with these outs."""
    n = ctypes.c_int64(0)
    c_outs = (ctypes.c_int64 * max(len(outs), 1))(*[int(o) for o in outs])
    _check(load_library().aqlm_lists_fused_workspace_bytes(len(outs), c_outs, 1, 16, 8, int(n_in), ctypes.byref(n)))
    return int(n.value)


def aqlm_linear_gemv_lists_fused(layers, x, ys=None, workspace=None):
    """[y_l] for layers l = (SliceLists, codebooks, scales) that all multiply x ([1][in]), in one launch."""
    n = len(layers)
    if not 1 <= n <= FUSED_MAX_LAYERS:
        raise ValueError(f"1 to {FUSED_MAX_LAYERS} layers")
    if not (x.is_cuda and x.is_contiguous() and x.dtype == torch.float16 and x.dim() == 2 and x.shape[0] <= 1):
        raise ValueError("x must be a contiguous float16 GPU tensor [1][in]")
    n_in, batch = int(x.shape[1]), int(x.shape[0])
    for lists, cb, s in layers:
        if lists.n_in != n_in:
            raise ValueError("every layer must take x's width")
        for name, t in (("codebooks", cb), ("scales", s)):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float16:
                raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
        if cb.shape != (1, 1 << 16, 8):
            raise ValueError("codebooks must be [1][65536][8]")
        if s.shape != (lists.out,):
            raise ValueError(f"scales must be [{lists.out}] (one per output row)")
        _same_device((("x", x), ("table", lists.table), ("entries", lists.entries), ("codebooks", cb),
                      ("scales", s)))
    outs = [lists.out for lists, _, _ in layers]
    if ys is None:
        ys = [torch.empty((batch, o), dtype=torch.float16, device=x.device) for o in outs]
    for y, o in zip(ys, outs):
        if y.shape != (batch, o) or y.dtype != torch.float16 or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous float16 [{batch}][{o}] tensor")
    if workspace is None:
        workspace = torch.empty(max(lists_fused_workspace_bytes(outs, n_in), 1), dtype=torch.uint8,
                                device=x.device)

    def arr(vals):
        return (ctypes.c_void_p * n)(*vals)
    i64 = ctypes.c_int64 * n
    _check(load_library().aqlm_linear_gemv_lists_fused(
        n, arr([l.table.data_ptr() for l, _, _ in layers]), arr([l.entries.data_ptr() for l, _, _ in layers]),
        i64(*[l.entries.numel() for l, _, _ in layers]), arr([cb.data_ptr() for _, cb, _ in layers]),
        arr([s.data_ptr() for _, _, s in layers]), i64(*outs), _ptr(x), arr([y.data_ptr() for y in ys]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), 1, 16, 8, n_in, batch, _stream(x.device)))
    return ys


def raw_call_fused(n_layers, codes, codebooks, scales, outs, x, ys, M, B, g, n_in, batch, stream=0) -> int:
    """Call aqlm_linear_gemv_fused with raw integer addresses (lists, or None for a NULL array)."""
    def arr(vals):
        return None if vals is None else (ctypes.c_void_p * max(len(vals), 1))(*vals)
    c_out = None if outs is None else (ctypes.c_int64 * max(len(outs), 1))(*outs)
    return int(load_library().aqlm_linear_gemv_fused(
        n_layers, arr(codes), arr(codebooks), arr(scales), c_out, ctypes.c_void_p(x), arr(ys),
        M, B, g, n_in, batch, ctypes.c_void_p(stream)))


def raw_call(fn_name, codes, codebooks, scales, x, y, M, B, g, out, n_in, batch, stream=0) -> int:
    """Call an entry point with raw integers/pointers and return its status (no checks)."""
    fn = getattr(load_library(), fn_name)
    return int(fn(ctypes.c_void_p(codes), ctypes.c_void_p(codebooks), ctypes.c_void_p(scales),
                  ctypes.c_void_p(x), ctypes.c_void_p(y), M, B, g, out, n_in, batch,
                  ctypes.c_void_p(stream)))
