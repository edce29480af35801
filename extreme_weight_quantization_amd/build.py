"""Build libaqlm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m extreme_weight_quantization_amd.build`` or call ``build()``.
Each source is compiled to an object file in parallel (under ``_build/`` at
the repository root), then the objects are linked into the library, which is
written next to this file so that it travels with the tree.  Every call
compiles every source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libaqlm.so")
OBJ_DIR = os.path.join(os.path.dirname(PKG_DIR), "_build")
SOURCES = ["aqlm_api.hip", "decode.hip", "gemv.hip", "gemm.hip", "gemm_pipe.hip", "generic.hip", "encode.hip",
           "gemv_lists.hip", "gemm_dense.hip", "gemv_stream.hip"]
ARCH = "gfx950"

# No fast-math and no flush-to-zero: decode must be bit-exact.  Packed fp32
# instructions are switched off for all device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, msgs


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(_run, cmds))
    for cmd, (rc, msgs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    rc, msgs = _run([cc, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
