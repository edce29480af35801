"""Repeats one library call on seeded synthetic inputs, for a profiler to watch.

    python3 -m extreme_weight_quantization_amd.profile_op OP SCHEME OUT IN [BATCH] [--reps N]

OP is gemv, gemm, gemm_dequant, decode or gemv_lists; SCHEME is 2x8, 1x16 or
an (M, B, g) triple written MxBgG (4x8g16).  OP copy runs a plain 64 MiB
device-to-device copy instead (the reference for scaling byte counters; the
other arguments are ignored).  Inputs follow the distributions of
the benchmark layers: codebooks N(0, 0.05) (2x8, other B = 8 schemes) or
N(0, 0.02) (1x16), uniform codes, scales U(0.5, 1.5), x N(0, 1).  The call
runs --reps times (default 5) after one untimed call, then the device is
synchronised; nothing is checked or printed but "done".  Under rocprofv3 the
kernel trace, statistics and counters of those calls are the profile of that
operation and shape.
"""
from __future__ import annotations

import argparse
import re


def parse_scheme(name: str):
    if name == "2x8":
        return 2, 8, 8, 0.05
    if name == "1x16":
        return 1, 16, 8, 0.02
    m = re.fullmatch(r"(\d+)x(\d+)g(\d+)", name)
    if not m:
        raise SystemExit(f"scheme {name!r}: 2x8, 1x16 or MxBgG")
    M, B, g = (int(v) for v in m.groups())
    return M, B, g, 0.05


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("op", choices=("gemv", "gemm", "gemm_dequant", "decode", "gemv_lists", "copy"))
    ap.add_argument("scheme")
    ap.add_argument("out", type=int)
    ap.add_argument("n_in", type=int)
    ap.add_argument("batch", type=int, nargs="?", default=1)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args(argv)

    import torch
    import extreme_weight_quantization_amd as E

    if not torch.cuda.is_available():
        raise SystemExit("profile_op needs a GPU")
    E.load_library()
    if args.op == "copy":
        src = torch.empty(32 << 20, dtype=torch.float16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(args.reps + 1):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    M, B, g, sd = parse_scheme(args.scheme)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    cb = (torch.randn((M, 1 << B, g), generator=gen, device="cuda") * sd).half()
    code_dtype = torch.uint8 if B <= 8 else torch.int16
    lo, hi = (-(1 << 15), 1 << 15) if B == 16 else (0, 1 << B)   # 16-bit codes stored as int16
    codes = torch.randint(lo, hi, (args.out, args.n_in // g, M), generator=gen, device="cuda", dtype=code_dtype)
    s = (torch.rand(args.out, generator=gen, device="cuda") + 0.5).half()
    x = torch.randn((args.batch, args.n_in), generator=gen, device="cuda").half()

    if args.op == "gemv":
        y = torch.empty((args.batch, args.out), dtype=torch.float16, device="cuda")
        call = lambda: E.aqlm_linear_gemv(codes, cb, s, x, y)
    elif args.op == "gemm":
        y = torch.empty((args.batch, args.out), dtype=torch.float16, device="cuda")
        call = lambda: E.aqlm_linear_gemm(codes, cb, s, x, y)
    elif args.op == "gemm_dequant":
        y = torch.empty((args.batch, args.out), dtype=torch.float16, device="cuda")
        ws = torch.empty((E.gemm_dequant_workspace_bytes(M, B, g, args.out, args.n_in),), dtype=torch.uint8,
                         device="cuda")
        call = lambda: E.aqlm_linear_gemm_dequant(codes, cb, s, x, y, ws)
    elif args.op == "decode":
        w = torch.empty((args.out, args.n_in), dtype=torch.float16, device="cuda")
        call = lambda: E.aqlm_linear_decode(codes, cb, s, w)
    else:
        if (M, B, g) != (1, 16, 8) or args.batch != 1:
            raise SystemExit("gemv_lists serves 1x16 at batch 1")
        lists = E.aqlm_lists_pack(codes)
        y = torch.empty((1, args.out), dtype=torch.float16, device="cuda")
        ws = torch.empty(E.lists_workspace_bytes(args.out, args.n_in), dtype=torch.uint8, device="cuda")
        call = lambda: E.aqlm_linear_gemv_lists(lists, cb, s, x, y, ws)
    call()
    torch.cuda.synchronize()
    for _ in range(args.reps):
        call()
    torch.cuda.synchronize()
    print("done", flush=True)


if __name__ == "__main__":
    main()
