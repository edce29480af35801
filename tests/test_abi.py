"""C-ABI library checks that need no GPU: the library loads, exports every
symbol that include/aqlm.h declares, and rejects bad arguments on the host
before any HIP call."""
import ctypes
import os
import re

import pytest

import extreme_weight_quantization_amd as E
from extreme_weight_quantization_amd import binding
from extreme_weight_quantization_amd.build import LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aqlm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build()
    return E.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aqlm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("aqlm_linear_gemv", "aqlm_linear_gemm", "aqlm_linear_decode"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in aqlm.h but not exported"
    assert set(declared_functions()) == set(binding.EXPORTED)


def test_exports_are_plain_c_symbols():
    out = os.popen(f"nm -D --defined-only {LIB_PATH}").read()
    exported = set(re.findall(r" T (aqlm_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for s in range(7):
        assert binding.status_str(s).startswith("AQLM_")
    assert "unknown" in binding.status_str(99)
    assert lib.aqlm_version().decode().count(".") == 2
    assert lib.aqlm_last_hip_error() == 0


A = 1 << 20  # a 16-byte aligned fake device address: validation never dereferences it

VALID = dict(codes=A, codebooks=A, scales=A, x=A, y=A, M=2, B=8, g=8, out=16, n_in=64, batch=1)


def call(fn, **kw):
    a = dict(VALID, **kw)
    return binding.raw_call(fn, a["codes"], a["codebooks"], a["scales"], a["x"], a["y"], a["M"],
                            a["B"], a["g"], a["out"], a["n_in"], a["batch"])


@pytest.mark.parametrize("fn", ["aqlm_linear_gemv", "aqlm_linear_gemm"])
def test_validation_product(lib, fn):
    assert call(fn, codes=0) == binding.AQLM_ERR_NULL
    assert call(fn, codebooks=0) == binding.AQLM_ERR_NULL
    assert call(fn, scales=0) == binding.AQLM_ERR_NULL
    assert call(fn, x=0) == binding.AQLM_ERR_NULL
    assert call(fn, y=0) == binding.AQLM_ERR_NULL
    for M, B, g in ((9, 8, 8), (0, 8, 8), (2, 17, 8), (1, 0, 8), (2, 8, 3), (1, 16, 64), (2, 8, 0)):
        assert call(fn, M=M, B=B, g=g) == binding.AQLM_ERR_SCHEME
    # any 1 <= M <= 8, 1 <= B <= 16, g in {1, 2, 4, 8, 16, 32} is a scheme (nothing enqueued: out = 0)
    for M, B, g in ((3, 8, 8), (2, 16, 8), (1, 8, 4), (8, 8, 32), (1, 16, 4), (1, 1, 1)):
        assert call(fn, M=M, B=B, g=g, out=0, n_in=64) == binding.AQLM_OK
    assert call(fn, M=1, B=8, g=32, n_in=48) == binding.AQLM_ERR_SHAPE   # in % g != 0
    assert call(fn, n_in=60) == binding.AQLM_ERR_SHAPE
    assert call(fn, n_in=0) == binding.AQLM_ERR_SHAPE
    assert call(fn, n_in=(1 << 20) + 8) == binding.AQLM_ERR_SHAPE
    assert call(fn, out=-1) == binding.AQLM_ERR_SHAPE
    assert call(fn, batch=-1) == binding.AQLM_ERR_SHAPE
    assert call(fn, out=1 << 31) == binding.AQLM_ERR_SHAPE
    assert call(fn, codes=A + 8) == binding.AQLM_ERR_ALIGN
    assert call(fn, x=A + 2) == binding.AQLM_ERR_ALIGN
    assert call(fn, y=A + 4) == binding.AQLM_ERR_ALIGN
    assert call(fn, codebooks=A + 8) == binding.AQLM_ERR_ALIGN
    assert call(fn, scales=A + 1) == binding.AQLM_ERR_ALIGN
    # empty problems enqueue nothing
    assert call(fn, out=0) == binding.AQLM_OK
    assert call(fn, batch=0) == binding.AQLM_OK


def test_validation_gemv_batch_limit(lib):
    assert call("aqlm_linear_gemv", batch=17) == binding.AQLM_ERR_SHAPE
    assert call("aqlm_linear_gemm", batch=17, out=0) == binding.AQLM_OK


def test_validation_decode(lib):
    assert call("aqlm_linear_decode", x=A) == binding.AQLM_ERR_NULL   # decode takes no x
    assert call("aqlm_linear_decode", x=0, y=0) == binding.AQLM_ERR_NULL
    assert call("aqlm_linear_decode", x=0, M=1, B=17) == binding.AQLM_ERR_SCHEME
    assert call("aqlm_linear_decode", x=0, n_in=12) == binding.AQLM_ERR_SHAPE
    assert call("aqlm_linear_decode", x=0, out=1 << 30, n_in=1 << 10) == binding.AQLM_ERR_SHAPE
    assert call("aqlm_linear_decode", x=0, y=A + 8) == binding.AQLM_ERR_ALIGN
    assert call("aqlm_linear_decode", x=0, out=0) == binding.AQLM_OK


def fused(n=3, **kw):
    a = dict(VALID, **kw)
    per = {k: kw.pop(k) for k in list(kw) if k.startswith("l_")}
    lists = {}
    for key in ("codes", "codebooks", "scales", "y"):
        vals = [a[key]] * n
        for (l, v) in per.get(f"l_{key}", []):
            vals[l] = v
        lists[key] = vals
    outs = [a["out"]] * n
    for (l, v) in per.get("l_out", []):
        outs[l] = v
    for key in ("codes", "codebooks", "scales", "y", "out"):
        if a.get(f"null_{key}"):
            lists[key] = None
            if key == "out":
                outs = None
    return binding.raw_call_fused(n, lists["codes"], lists["codebooks"], lists["scales"], outs, a["x"],
                                  lists["y"], a["M"], a["B"], a["g"], a["n_in"], a["batch"])


def test_validation_gemv_fused(lib):
    assert fused(n=0) == binding.AQLM_ERR_SHAPE
    assert fused(n=binding.FUSED_MAX_LAYERS + 1) == binding.AQLM_ERR_SHAPE
    for key in ("codes", "codebooks", "scales", "y", "out"):
        assert fused(**{f"null_{key}": True}) == binding.AQLM_ERR_NULL
    # every layer is validated like aqlm_linear_gemv; the first failure is returned
    assert fused(l_codes=[(1, 0)]) == binding.AQLM_ERR_NULL
    assert fused(l_scales=[(2, A + 1)]) == binding.AQLM_ERR_ALIGN
    assert fused(l_y=[(0, A + 8)], l_codes=[(2, 0)]) == binding.AQLM_ERR_ALIGN
    assert fused(l_out=[(1, -1)]) == binding.AQLM_ERR_SHAPE
    assert fused(x=0) == binding.AQLM_ERR_NULL
    assert fused(batch=17) == binding.AQLM_ERR_SHAPE
    assert fused(M=1, B=17) == binding.AQLM_ERR_SCHEME
    # empty layers are skipped; an all-empty call enqueues nothing
    assert fused(out=0) == binding.AQLM_OK
    assert fused(out=0, l_codes=[(0, 0)]) == binding.AQLM_OK
    assert fused(batch=0) == binding.AQLM_OK


def enc(**kw):
    a = dict(w=A, scales=A, codebooks=A, codes=A, M=2, B=8, g=8, out=16, n_in=64)
    a.update(kw)
    return int(lib_fn("aqlm_encode_greedy")(a["w"], a["scales"], a["codebooks"], a["codes"], a["M"], a["B"], a["g"],
                                            a["out"], a["n_in"], None))


def km(**kw):
    a = dict(w=A, scales=A, seeds=A, codebooks=A, codes=A, ws=A, ws_bytes=1 << 30, M=2, B=8, g=8, out=16, n_in=64,
             iters=3)
    a.update(kw)
    return int(lib_fn("aqlm_kmeans_init")(a["w"], a["scales"], a["seeds"], a["codebooks"], a["codes"], a["ws"],
                                          a["ws_bytes"], a["M"], a["B"], a["g"], a["out"], a["n_in"], a["iters"], None))


def lib_fn(name):
    return getattr(E.load_library(), name)


def test_kmeans_workspace_bytes(lib):
    import ctypes as C
    n = C.c_int64(0)
    assert lib.aqlm_kmeans_workspace_bytes(2, 8, 8, C.byref(n)) == binding.AQLM_OK
    assert n.value == 256 * 8 * 8 + 256 * 8 + 256 * 8 * 4 + 16   # int64 sums, int64 counts, fp32 centroids, flag
    assert lib.aqlm_kmeans_workspace_bytes(1, 16, 8, C.byref(n)) == binding.AQLM_OK
    assert n.value == 65536 * (8 * 12 + 8) + 16
    assert lib.aqlm_kmeans_workspace_bytes(2, 17, 8, C.byref(n)) == binding.AQLM_ERR_SCHEME
    assert lib.aqlm_kmeans_workspace_bytes(2, 8, 8, None) == binding.AQLM_ERR_NULL
    assert binding.kmeans_workspace_bytes(4, 8, 16) == 256 * (16 * 12 + 8) + 16


def test_validation_encode(lib):
    for key in ("w", "scales", "codebooks", "codes"):
        assert enc(**{key: 0}) == binding.AQLM_ERR_NULL
    assert enc(M=9) == binding.AQLM_ERR_SCHEME
    assert enc(g=3) == binding.AQLM_ERR_SCHEME
    assert enc(n_in=60) == binding.AQLM_ERR_SHAPE
    assert enc(out=-1) == binding.AQLM_ERR_SHAPE
    assert enc(w=A + 8) == binding.AQLM_ERR_ALIGN
    assert enc(codes=A + 2) == binding.AQLM_ERR_ALIGN
    assert enc(scales=A + 1) == binding.AQLM_ERR_ALIGN
    assert enc(out=0, w=0) == binding.AQLM_OK


def test_validation_kmeans(lib):
    for key in ("w", "scales", "codebooks", "codes", "seeds", "ws"):
        assert km(**{key: 0}) == binding.AQLM_ERR_NULL
    assert km(B=0) == binding.AQLM_ERR_SCHEME
    assert km(iters=-1) == binding.AQLM_ERR_SHAPE
    assert km(iters=10001) == binding.AQLM_ERR_SHAPE
    assert km(ws_bytes=256 * (8 * 12 + 8) - 1) == binding.AQLM_ERR_SHAPE
    assert km(seeds=A + 4) == binding.AQLM_ERR_ALIGN
    assert km(ws=A + 8) == binding.AQLM_ERR_ALIGN
    assert km(out=0, seeds=0, ws=0) == binding.AQLM_OK


def test_binding_rejects_cpu_tensors(lib):
    import torch
    codes = torch.zeros((4, 8, 2), dtype=torch.uint8)
    cb = torch.zeros((2, 256, 8), dtype=torch.float16)
    s = torch.ones(4, dtype=torch.float16)
    x = torch.zeros((1, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        E.aqlm_linear_gemv(codes, cb, s, x)
    with pytest.raises(ValueError):
        E.aqlm_linear_decode(codes, cb, s)


# --------------------------------------------------------------------------
# 1x16 slice lists


def lists_geometry_sizes(out, n_in):
    """Table and workspace bytes from the layout's definition (tiles of 64 rows, blocks of <= 1024 groups)."""
    G = n_in // 8
    J = -(-G // 1024)
    n_rt = -(-out // 64)
    return (2 * 8 * J * n_rt + 2) * 4, 8 * J * n_rt * 64 * 4


@pytest.mark.parametrize("out,n_in", [(4096, 4096), (11008, 4096), (4096, 11008), (28672, 8192), (8192, 28672),
                                      (1024, 8192), (1, 8), (130, 72), (0, 64)])
def test_lists_sizes(lib, out, n_in):
    table, ws = lists_geometry_sizes(out, n_in)
    assert binding.lists_table_bytes(out, n_in) == table
    assert binding.lists_workspace_bytes(out, n_in) == ws


def test_lists_size_validation(lib):
    import ctypes as C
    n = C.c_int64(0)
    for name in ("aqlm_lists_table_bytes", "aqlm_lists_workspace_bytes"):
        fn = lib_fn(name)
        assert fn(1, 16, 8, 64, 512, C.byref(n)) == binding.AQLM_OK
        assert fn(2, 8, 8, 64, 512, C.byref(n)) == binding.AQLM_ERR_SCHEME
        assert fn(1, 16, 4, 64, 512, C.byref(n)) == binding.AQLM_ERR_SCHEME
        assert fn(1, 16, 8, 64, 500, C.byref(n)) == binding.AQLM_ERR_SHAPE
        assert fn(1, 16, 8, 64, 0, C.byref(n)) == binding.AQLM_ERR_SHAPE
        assert fn(1, 16, 8, -1, 512, C.byref(n)) == binding.AQLM_ERR_SHAPE
        assert fn(1, 16, 8, (1 << 30) + 1, 8, C.byref(n)) == binding.AQLM_ERR_SHAPE
        assert fn(1, 16, 8, 1 << 20, 1 << 19, C.byref(n)) == binding.AQLM_ERR_SHAPE   # 2^36 codes
        assert fn(1, 16, 8, 64, 512, None) == binding.AQLM_ERR_NULL


def lists_gemv(**kw):
    a = dict(table=A, entries=A, entries_bytes=1 << 20, cb=A, scales=A, x=A, y=A, ws=A, ws_bytes=1 << 30,
             M=1, B=16, g=8, out=64, n_in=512, batch=1)
    a.update(kw)
    return int(lib_fn("aqlm_linear_gemv_lists")(a["table"], a["entries"], a["entries_bytes"], a["cb"], a["scales"],
                                                a["x"], a["y"], a["ws"], a["ws_bytes"], a["M"], a["B"], a["g"],
                                                a["out"], a["n_in"], a["batch"], None))


def test_validation_gemv_lists(lib):
    for key in ("table", "entries", "cb", "scales", "x", "y", "ws"):
        assert lists_gemv(**{key: 0}) == binding.AQLM_ERR_NULL
    assert lists_gemv(M=2, B=8) == binding.AQLM_ERR_SCHEME
    assert lists_gemv(batch=2) == binding.AQLM_ERR_SHAPE
    assert lists_gemv(batch=-1) == binding.AQLM_ERR_SHAPE
    assert lists_gemv(n_in=520 + 4) == binding.AQLM_ERR_SHAPE
    assert lists_gemv(entries_bytes=-1) == binding.AQLM_ERR_SHAPE
    assert lists_gemv(ws_bytes=lists_geometry_sizes(64, 512)[1] - 1) == binding.AQLM_ERR_SHAPE
    for key in ("table", "entries", "cb", "x", "y", "ws"):
        assert lists_gemv(**{key: A + 8}) == binding.AQLM_ERR_ALIGN
    assert lists_gemv(scales=A + 1) == binding.AQLM_ERR_ALIGN
    assert lists_gemv(batch=0, table=0, entries=0, x=0, y=0) == binding.AQLM_OK
    assert lists_gemv(out=0, table=0, ws=0) == binding.AQLM_OK


def test_validation_lists_plan_and_fill(lib):
    plan, fill = lib_fn("aqlm_lists_plan"), lib_fn("aqlm_lists_fill")
    assert plan(A, None, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_NULL
    assert plan(None, A, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_NULL
    assert plan(A, A + 8, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_ALIGN
    assert plan(A, A, 2, 8, 8, 64, 512, None) == binding.AQLM_ERR_SCHEME
    assert plan(A, A, 1, 16, 8, 64, 12, None) == binding.AQLM_ERR_SHAPE
    for args in ((None, A, A), (A, None, A), (A, A, None)):
        assert fill(*args, 1 << 20, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_NULL
    assert fill(A, A, A + 4, 1 << 20, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_ALIGN
    assert fill(A, A, A, -1, 1, 16, 8, 64, 512, None) == binding.AQLM_ERR_SHAPE
    assert fill(A, A, A, 1 << 20, 1, 12, 4, 64, 512, None) == binding.AQLM_ERR_SCHEME
    assert fill(None, None, None, 0, 1, 16, 8, 0, 512, None) == binding.AQLM_OK


def test_binding_lists_rejects_bad_codes(lib):
    import torch
    with pytest.raises(ValueError):
        E.aqlm_lists_pack(torch.zeros((4, 8, 1), dtype=torch.int16))           # CPU tensor


def lists_fused(n=2, **kw):
    a = dict(tables=[A] * n, entries=[A] * n, eb=[1 << 20] * n, cbs=[A] * n, scales=[A] * n, outs=[64] * n, x=A,
             ys=[A] * n, ws=A, ws_bytes=1 << 30, M=1, B=16, g=8, n_in=512, batch=1)
    a.update(kw)
    import ctypes as C

    def arr(v):
        return None if v is None else (C.c_void_p * max(len(v), 1))(*v)

    def i64(v):
        return None if v is None else (C.c_int64 * max(len(v), 1))(*v)
    return int(lib_fn("aqlm_linear_gemv_lists_fused")(
        n, arr(a["tables"]), arr(a["entries"]), i64(a["eb"]), arr(a["cbs"]), arr(a["scales"]), i64(a["outs"]),
        a["x"], arr(a["ys"]), a["ws"], a["ws_bytes"], a["M"], a["B"], a["g"], a["n_in"], a["batch"], None))


def test_validation_gemv_lists_fused(lib):
    for key in ("tables", "entries", "eb", "cbs", "scales", "outs", "ys"):
        assert lists_fused(**{key: None}) == binding.AQLM_ERR_NULL
    assert lists_fused(n=0) == binding.AQLM_ERR_SHAPE
    assert lists_fused(n=9) == binding.AQLM_ERR_SHAPE
    assert lists_fused(tables=[A, 0]) == binding.AQLM_ERR_NULL
    assert lists_fused(x=0) == binding.AQLM_ERR_NULL
    assert lists_fused(ws=0) == binding.AQLM_ERR_NULL
    assert lists_fused(M=2, B=8) == binding.AQLM_ERR_SCHEME
    assert lists_fused(batch=2) == binding.AQLM_ERR_SHAPE
    assert lists_fused(outs=[64, -1]) == binding.AQLM_ERR_SHAPE
    assert lists_fused(eb=[1 << 20, -1]) == binding.AQLM_ERR_SHAPE
    assert lists_fused(entries=[A, A + 4]) == binding.AQLM_ERR_ALIGN
    assert lists_fused(ws=A + 8) == binding.AQLM_ERR_ALIGN
    one = lists_geometry_sizes(64, 512)[1]
    assert lists_fused(ws_bytes=2 * one - 1) == binding.AQLM_ERR_SHAPE          # 2 x 16 KB, 256-aligned
    assert lists_fused(outs=[0, 0], tables=[0, 0], x=0, ws=0) == binding.AQLM_OK
    assert lists_fused(batch=0, x=0, ws=0) == binding.AQLM_OK


def test_lists_fused_workspace_bytes(lib):
    one = lambda o, i: -(-lists_geometry_sizes(o, i)[1] // 256) * 256
    assert binding.lists_fused_workspace_bytes([4096, 4096, 4096], 4096) == 3 * one(4096, 4096)
    assert binding.lists_fused_workspace_bytes([11008, 0, 100], 4096) == one(11008, 4096) + one(100, 4096)
    with pytest.raises(ValueError):
        binding.lists_fused_workspace_bytes([], 4096)
    with pytest.raises(ValueError):
        binding.lists_fused_workspace_bytes([64], 4100)


def dequant(**kw):
    a = dict(VALID, ws=A, ws_bytes=16 * 64 * 2)
    a.update(kw)
    return int(lib_fn("aqlm_linear_gemm_dequant")(a["codes"], a["codebooks"], a["scales"], a["x"], a["y"], a["ws"],
                                                  a["ws_bytes"], a["M"], a["B"], a["g"], a["out"], a["n_in"],
                                                  a["batch"], None))


def test_validation_gemm_dequant(lib):
    for key in ("codes", "codebooks", "scales", "x", "y", "ws"):
        assert dequant(**{key: 0}) == binding.AQLM_ERR_NULL
    assert dequant(M=9) == binding.AQLM_ERR_SCHEME
    assert dequant(ws_bytes=16 * 64 * 2 - 1) == binding.AQLM_ERR_SHAPE
    assert dequant(n_in=60) == binding.AQLM_ERR_SHAPE
    assert dequant(batch=-1) == binding.AQLM_ERR_SHAPE
    assert dequant(out=1 << 24, n_in=4096, ws_bytes=1 << 40) == binding.AQLM_ERR_SHAPE   # out * in / g >= 2^32
    for key in ("codes", "codebooks", "x", "y", "ws"):
        assert dequant(**{key: A + 8}) == binding.AQLM_ERR_ALIGN
    assert dequant(scales=A + 1) == binding.AQLM_ERR_ALIGN
    # empty problems enqueue nothing and need no workspace
    assert dequant(out=0, ws=0, ws_bytes=0) == binding.AQLM_OK
    assert dequant(batch=0, ws=0, ws_bytes=0) == binding.AQLM_OK


def test_gemm_dequant_workspace_bytes(lib):
    assert binding.gemm_dequant_workspace_bytes(2, 8, 8, 4096, 4096) == 4096 * 4096 * 2
    assert binding.gemm_dequant_workspace_bytes(1, 16, 8, 11008, 4096) == 11008 * 4096 * 2
    assert binding.gemm_dequant_workspace_bytes(2, 8, 8, 100, 520) == 0      # in % 64 != 0: not used
    assert binding.gemm_dequant_workspace_bytes(4, 8, 16, 0, 64) == 0
    n = ctypes.c_int64(0)
    fn = lib_fn("aqlm_gemm_dequant_workspace_bytes")
    assert fn(9, 8, 8, 64, 64, ctypes.byref(n)) == binding.AQLM_ERR_SCHEME
    assert fn(2, 8, 8, -1, 64, ctypes.byref(n)) == binding.AQLM_ERR_SHAPE
    assert fn(2, 8, 8, 64, 60, ctypes.byref(n)) == binding.AQLM_ERR_SHAPE
    assert fn(2, 8, 8, 64, 64, None) == binding.AQLM_ERR_NULL
