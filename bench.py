#!/usr/bin/env python3
"""Benchmark of the AQLM 2-bit quantized linear layer on one MI355X.

Headline workload: the seven projections of one Llama-2-7B decoder block
(q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008) as AQLM 1x16
(one 65536-entry fp16 codebook, int16 codes, g = 8) decode-phase GEMVs at
batch 1.  One step runs all seven layers once, each as one
aqlm_linear_gemv_lists call over the layer's slice lists (its codes regrouped
by codebook slice once, at load time, before any timed region).  The reported
value is the achieved HBM bandwidth over the counted bytes (codes at 2 bits
per weight + scales + activations + outputs), with inputs resident in HBM and
rotated over enough distinct buffer sets to defeat the 256 MB last-level
cache.

Also measured in the same run (reported under "breakdown", not in value): the
same block with the codes in their stored layout (aqlm_linear_gemv, per-code
codebook gathers), alone and with q,k,v and gate,up fused; 2x8 GEMV at batch
1/4/16 on the same block; the Llama-2-70B 1x16 layers at batch 1 in both
layouts; the 70B layers as 2x8 at batch 1, alone, in aggregate and as a block
step with q,k,v and gate,up fused; the 2048-token prefill GEMM on the 7B shapes (both schemes); the
standalone decode kernel; the other 2-bit schemes; the encoder; and the fp16
comparator.  Secondary figures: the headline as a share of a measured
device-to-device copy's bandwidth, the effective weight rate (fp16-equivalent
weight bytes 2 out in per second: a reading of a term the pages leave
undefined), and, not counted, the same step with one buffer set reused (codes
resident in the last-level cache).  The CPU oracle is timed on the host over
whole block steps, with the CPU model, the BLAS numpy uses and the share of
its time spent decoding.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import copy
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
# fp32 vector ALU: 157.3 TFLOP/s counts a fused multiply-add as 2 flops, so a
# plain (unfused) add, subtract or multiply peaks at half that op rate.
VALU_F32_PEAK_TOPS = 157.3 / 2.0
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
# Seconds of untimed replays before each breakdown measurement.  The GPU clock falls
# when the device idles (host-side setup between measurements) and takes tens of
# milliseconds of load to climb back: timed cold, a 10-launch prefill measurement
# ran 5-10 % slower than the same launches in steady state.
WARM_S = 0.25

BLOCK_7B = ((4096, 4096),) * 4 + ((11008, 4096),) * 2 + ((4096, 11008),)
SHAPES_7B = ((4096, 4096), (11008, 4096), (4096, 11008))
SHAPES_70B = ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672))
# A Llama-2-70B decoder block in the same order as BLOCK_7B: q, k, v (GQA), o, gate, up, down.
BLOCK_70B = ((8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192), (28672, 8192), (8192, 28672))
SCHEMES = {"2x8": (2, 8, 8, 0.05), "1x16": (1, 16, 8, 0.02)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(out, n_in, batch):
    """Counted bytes of one GEMV: codes (2 bits/weight) + scales + x + y."""
    return out * n_in // 4 + 2 * out + 2 * n_in * batch + 2 * out * batch


# ----------------------------------------------------------------------------
# Synthetic layers on the GPU (seeded torch generator; same distributions as
# extreme_weight_quantization_amd.synth, drawn on the device for speed).


def make_codebooks(torch, scheme, gen):
    M, B, g, sigma = SCHEMES[scheme]
    cb = torch.randn((M, 1 << B, g), generator=gen, device="cuda", dtype=torch.float32) * sigma
    return cb.half()


def make_codes(torch, scheme, out, n_in, gen):
    M, B, g, _ = SCHEMES[scheme]
    if B == 8:
        return torch.randint(0, 256, (out, n_in // g, M), generator=gen, device="cuda", dtype=torch.uint8)
    return torch.randint(-32768, 32768, (out, n_in // g, M), generator=gen, device="cuda", dtype=torch.int16)


def make_generic(torch, M, B, g, out, n_in, gen, sigma=0.05):
    """Codebooks and codes of any (M, B, g): codes uniform over the 2^B indices, in whole bytes."""
    cb = (torch.randn((M, 1 << B, g), generator=gen, device="cuda", dtype=torch.float32) * sigma).half()
    c = torch.randint(0, 1 << B, (out, n_in // g, M), generator=gen, device="cuda", dtype=torch.int32)
    codes = c.to(torch.uint8) if B <= 8 else c.to(torch.int16)
    return cb, codes


def generic_gemv_bytes(M, B, g, out, n_in, batch):
    """Counted bytes of one GEMV of any scheme: codes (M codes of 1 or 2 bytes per group) + scales + x + y."""
    return out * (n_in // g) * M * (1 if B <= 8 else 2) + 2 * out + 2 * n_in * batch + 2 * out * batch


# The budget-equivalent 2-bit schemes of "Key AQLM quantization parameters" at B = 8.
GENERIC_2BIT = ((1, 8, 4), (4, 8, 16), (8, 8, 32))


def make_scales(torch, out, gen):
    return (torch.rand(out, generator=gen, device="cuda") + 0.5).half()


def make_x(torch, batch, n_in, gen):
    return torch.randn((batch, n_in), generator=gen, device="cuda").half()


class LayerSet:
    """n_sets distinct copies of codes+scales (+x, y) for a list of layer shapes."""

    def __init__(self, torch, scheme, shapes, batch, n_sets, seed=0):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        self.scheme, self.shapes, self.batch = scheme, shapes, batch
        self.cb = make_codebooks(torch, scheme, gen)
        self.sets = []
        for _ in range(n_sets):
            layers = []
            for out, n_in in shapes:
                layers.append((make_codes(torch, scheme, out, n_in, gen), make_scales(torch, out, gen),
                               make_x(torch, batch, n_in, gen),
                               torch.empty((batch, out), dtype=torch.float16, device="cuda")))
            self.sets.append(layers)
        self.bytes_per_step = sum(gemv_bytes(o, i, batch) for o, i in shapes)
        self.lists = None

    def pack_lists(self, torch, E):
        """Slice lists of every 1x16 layer (the load-time regrouping; never inside a timed region)."""
        self.lists = [[E.aqlm_lists_pack(codes) for (codes, _, _, _) in layers] for layers in self.sets]
        # one workspace for single calls and for the fused groups of the 7B block (the largest need)
        need = max(E.lists_workspace_bytes(o, i) for o, i in self.shapes)
        if self.shapes == BLOCK_7B:
            need = max([need] + [E.lists_fused_workspace_bytes([self.shapes[i][0] for i in grp], self.shapes[grp[0]][1])
                                 for grp in BLOCK_7B_GROUPS])
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        return sum(l.entries.numel() for l in self.lists[0])


def sets_needed(shapes, batch, min_bytes=4 * LLC_BYTES, cap=64):
    per = sum(gemv_bytes(o, i, batch) for o, i in shapes)
    return max(2, min(cap, -(-min_bytes // per)))


# ----------------------------------------------------------------------------


def capture(torch, launches):
    """A HIP graph of the given launch closures (run once eagerly first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in launches:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    torch.cuda.synchronize()
    return g


def warm(torch, graph, secs=WARM_S):
    """Replays `graph` (untimed) until the device has been busy for `secs` seconds."""
    t0 = time.perf_counter()
    while True:
        graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= secs:
            return


def replay_us(torch, graph, reps=1):
    """Wall time on the device of `reps` replays of `graph`, in microseconds (HIP events)."""
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3


def gemv_launches(E, ls, k0, n_steps, only=None, lists=False):
    out = []
    for k in range(k0, k0 + n_steps):
        for li, (codes, s, x, y) in enumerate(ls.sets[k % len(ls.sets)]):
            if only is None or ls.shapes[li] == only:
                if lists:
                    lst = ls.lists[k % len(ls.sets)][li]
                    out.append(lambda l=lst, s=s, x=x, y=y: E.aqlm_linear_gemv_lists(l, ls.cb, s, x, y, ls.ws))
                else:
                    out.append(lambda c=codes, s=s, x=x, y=y: E.aqlm_linear_gemv(c, ls.cb, s, x, y))
    return out


# The 7B block's layers that multiply the same activations: q, k, v | o | gate, up | down.
BLOCK_7B_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))


def fused_block_launches(E, ls, k0, n_steps, lists=False):
    """One pass over the block per step with the projections that share x fused into one launch."""
    out = []
    for k in range(k0, k0 + n_steps):
        layers = ls.sets[k % len(ls.sets)]
        for grp in BLOCK_7B_GROUPS:
            x = layers[grp[0]][2]
            if lists:
                lst = ls.lists[k % len(ls.sets)]
                if len(grp) == 1:
                    _, s, _, y = layers[grp[0]]
                    out.append(lambda l=lst[grp[0]], s=s, x=x, y=y: E.aqlm_linear_gemv_lists(l, ls.cb, s, x, y, ls.ws))
                else:
                    lay = [(lst[i], ls.cb, layers[i][1]) for i in grp]
                    ys = [layers[i][3] for i in grp]
                    out.append(lambda lay=lay, x=x, ys=ys: E.aqlm_linear_gemv_lists_fused(lay, x, ys, ls.ws))
            elif len(grp) == 1:
                codes, s, _, y = layers[grp[0]]
                out.append(lambda c=codes, s=s, x=x, y=y: E.aqlm_linear_gemv(c, ls.cb, s, x, y))
            else:
                lay = [(layers[i][0], ls.cb, layers[i][1]) for i in grp]
                ys = [layers[i][3] for i in grp]
                out.append(lambda lay=lay, x=x, ys=ys: E.aqlm_linear_gemv_fused(lay, x, ys))
    return out


def time_fused_block(torch, E, ls: LayerSet, steps, warmup, lists=False):
    """ms per 7B block step with fused projections (same rotation and graph timing as time_gemv,
    after WARM_S seconds of untimed replays)."""
    g_warm = capture(torch, fused_block_launches(E, ls, 0, max(1, warmup), lists))
    g_main = capture(torch, fused_block_launches(E, ls, warmup, steps, lists))
    replay_us(torch, g_warm)
    warm(torch, g_main)
    ms_step = replay_us(torch, g_main) / steps / 1e3
    del g_warm, g_main
    return ms_step


def time_gemv(torch, E, ls: LayerSet, steps, warmup, lists=False, warm_s=WARM_S):
    """Times exactly `steps` passes over the layer list (rotating buffer sets).

    The launches are captured in a HIP graph so that the device runs them
    back to back; the timed region is one replay of that graph between two
    HIP events, after one replay of `warmup` steps and `warm_s` seconds of
    untimed replays of the timed graph (0 for the headline: exactly `warmup`
    steps).  Per-shape kernel durations come from graphs of back-to-back
    launches of one shape, each after WARM_S seconds of untimed replays.
    Returns (ms per step, {shape: us per launch}).
    """
    g_warm = capture(torch, gemv_launches(E, ls, 0, max(1, warmup), lists=lists))
    g_main = capture(torch, gemv_launches(E, ls, warmup, steps, lists=lists))
    replay_us(torch, g_warm)
    if warm_s > 0:
        warm(torch, g_main, warm_s)
    ms_step = replay_us(torch, g_main) / steps / 1e3
    per_shape = {}
    for shape in dict.fromkeys(ls.shapes):
        n = max(1, min(len(ls.sets), 64))
        g = capture(torch, gemv_launches(E, ls, 0, n, only=shape, lists=lists))
        count = n * ls.shapes.count(shape)
        warm(torch, g)
        per_shape[shape] = replay_us(torch, g, reps=4) / (4 * count)
        del g
    del g_warm, g_main
    return ms_step, per_shape


def hbm_copy_gbps(torch, mib=512, reps=10):
    """Read + write bytes per second of a plain device-to-device copy (the measured
    streaming bandwidth the GEMV rates are also compared with)."""
    src = torch.empty(mib << 19, dtype=torch.float16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbps = 2 * (mib << 20) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def time_calls(torch, launch, iters, warmup):
    """Mean us per launch of `launch(i)` over `iters` back-to-back launches in a HIP graph
    (after `warmup` eager launches and WARM_S seconds of untimed replays)."""
    for i in range(warmup):
        launch(i)
    g = capture(torch, [lambda i=i: launch(i) for i in range(iters)])
    warm(torch, g)
    us = replay_us(torch, g, reps=3) / (3 * iters)
    del g
    return us


def spot_check(torch, E, ls: LayerSet, rows_per_layer=32, lists=False):
    """Compares sampled outputs of set 0 with the CPU oracle (parity of the timed launches)."""
    from oracle import aqlm_oracle as O
    worst = 0.0
    cb = ls.cb.cpu().numpy()
    for li, (codes, s, x, y) in enumerate(ls.sets[0]):
        if lists:
            E.aqlm_linear_gemv_lists(ls.lists[0][li], ls.cb, s, x, y, ls.ws)
        else:
            E.aqlm_linear_gemv(codes, ls.cb, s, x, y)
        torch.cuda.synchronize()
        out = codes.shape[0]
        rows = np.unique(np.linspace(0, out - 1, rows_per_layer).astype(np.int64))
        yr = O.linear_ref_rows_f64(codes.cpu().numpy(), cb, s.cpu().numpy(), x.cpu().numpy(), rows)
        rel, mx, ref_max = O.parity_errors(y.cpu().numpy().astype(np.float64)[:, rows], yr)
        if not (rel <= 1e-3 and mx <= 1e-2 * ref_max):
            raise RuntimeError(f"parity check failed: rel {rel:.3e} max {mx:.3e}")
        worst = max(worst, rel)
    return worst


def recorded_traffic(record="gemv_lists_1x16_llama2_7b_block_b1_traffic.json",
                     sources=("gemv_lists.hip", "aqlm_device.h")):
    """Per-launch HBM bytes of the headline kernels from a committed rocprofv3 PMC record.

    Returned only while the kernel sources hash to the value recorded with the
    counters; a changed kernel reports None until the counters are taken again.
    """
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    rec_path = os.path.join(root, "profiles", record)
    try:
        rec = json.load(open(rec_path))
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(root, "extreme_weight_quantization_amd", "csrc", f), "rb").read())
        if h.hexdigest()[:16] != rec["source_sha256_16"]:
            return None
        return rec["per_launch_traffic_bytes_mean"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(min_seconds=10.0):
    """The CPU oracle (decode in fp32, float64 product) over the headline step, 1x16, batch 1.

    Runs whole 7-layer 7B block steps (one drawn layer per shape, reused) until
    at least `min_seconds` of oracle time have passed, and reports the
    counted bytes per second of oracle time."""
    from extreme_weight_quantization_amd import synth
    from oracle import aqlm_oracle as O
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    layers = {shape: synth.make_layer("1x16", shape[0], shape[1], batch=1, seed=0) for shape in SHAPES_7B}
    nbytes, elapsed, steps = 0, 0.0, 0
    while elapsed < min_seconds:
        for shape in BLOCK_7B:
            L = layers[shape]
            t = time.perf_counter()
            O.linear_ref_f64(L.codes, L.codebooks, L.scales, L.x)
            elapsed += time.perf_counter() - t
            nbytes += gemv_bytes(shape[0], shape[1], 1)
        steps += 1
    # the oracle's fp32 decode alone, once per layer of a step (the rest of its time is the product)
    dec = 0.0
    for shape in BLOCK_7B:
        L = layers[shape]
        t = time.perf_counter()
        O.decode_fp32(L.codes, L.codebooks, L.scales)
        dec += time.perf_counter() - t
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:  # pragma: no cover
        pass
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"numpy oracle (fp32 decode + float64 product) on {steps} Llama-2-7B block steps "
                      f"(7 AQLM 1x16 layers each, batch 1): {elapsed:.1f} s for {nbytes / 1e6:.1f} MB "
                      "counted bytes",
            "us_per_layer": round(elapsed / (7 * steps) * 1e6, 1),
            "decode_share": round(dec / (elapsed / steps), 3),
            "cpu_model": cpu_model, "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only, no breakdown or CPU leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle leg")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 64 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; layers would shard by "
              "output rows with nothing exchanged (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import extreme_weight_quantization_amd as E
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    E.load_library()
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)

    # ---- headline: 7B block, 1x16, batch 1, codes as slice lists -----------
    n_sets = sets_needed(BLOCK_7B, 1)
    ls = LayerSet(torch, "1x16", BLOCK_7B, 1, n_sets, seed=0)
    entry_bytes_step = ls.pack_lists(torch, E)
    worst = spot_check(torch, E, ls, lists=True)
    torch.cuda.synchronize()
    ms_step, shape_us = time_gemv(torch, E, ls, args.steps, args.warmup, lists=True, warm_s=0)
    value = ls.bytes_per_step / (ms_step * 1e-3) / 1e9
    kern_us_step = sum(shape_us[sh] for sh in BLOCK_7B)
    achieved = ls.bytes_per_step / (kern_us_step * 1e-6) / 1e9

    def shape_table(su, batch=1):
        return {f"{o}x{i}": {"us": round(us, 3), "GBps": round(gemv_bytes(o, i, batch) / (us * 1e-6) / 1e9, 1),
                             "pct_hbm_peak": round(100 * gemv_bytes(o, i, batch) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                             "effective_weight_GBps": round(2 * o * i / (us * 1e-6) / 1e9, 1)}
                for (o, i), us in su.items()}

    per_shape = shape_table(shape_us)
    breakdown = {"gemv_1x16_b1_7b": per_shape}
    copy_gbps = hbm_copy_gbps(torch)
    breakdown["hbm_copy"] = {"GBps": round(copy_gbps, 1),
                             "what": "torch device-to-device copy of 512 MiB, read + write bytes per second"}
    fused = {}
    if not args.quick:
        # not counted: one buffer set reused every step, so the codes stay in the last-level cache
        hot = copy.copy(ls)
        hot.sets, hot.lists = ls.sets[:1], ls.lists[:1]
        ms_hot, _ = time_gemv(torch, E, hot, args.steps, args.warmup, lists=True)
        breakdown["gemv_1x16_b1_7b_hot_single_set"] = {
            "ms_per_step": round(ms_hot, 5), "GBps_step": round(ls.bytes_per_step / (ms_hot * 1e-3) / 1e9, 1),
            "note": "not counted: the same buffers every step (resident in the 256 MB last-level cache)"}
        del hot
        # the same layers and buffers with the codes in their stored layout (per-code L2 gathers)
        worst_plain = spot_check(torch, E, ls)
        ms_plain, shape_plain = time_gemv(torch, E, ls, args.steps, args.warmup)
        kp = sum(shape_plain[sh] for sh in BLOCK_7B)
        breakdown["gemv_1x16_b1_7b_stored_layout"] = {
            "ms_per_step": round(ms_plain, 5), "us_per_layer": round(ms_plain * 1e3 / len(BLOCK_7B), 3),
            "GBps_step": round(ls.bytes_per_step / (ms_plain * 1e-3) / 1e9, 1),
            "GBps_kernel": round(ls.bytes_per_step / (kp * 1e-6) / 1e9, 1),
            "spot_check_rel_l2": worst_plain, "per_shape": shape_table(shape_plain)}
        ms_fl = time_fused_block(torch, E, ls, max(20, args.steps // 2), 5, lists=True)
        fused["1x16_b1"] = {"ms_per_step": round(ms_fl, 5), "us_per_layer": round(ms_fl * 1e3 / len(BLOCK_7B), 3),
                            "GBps_step": round(ls.bytes_per_step / (ms_fl * 1e-3) / 1e9, 1),
                            "unfused_ms_per_step": round(ms_step, 5), "codes_layout": "slice lists"}
        ms_f = time_fused_block(torch, E, ls, max(20, args.steps // 2), 5)
        fused["1x16_b1_stored_layout"] = {"ms_per_step": round(ms_f, 5),
                                          "us_per_layer": round(ms_f * 1e3 / len(BLOCK_7B), 3),
                                          "GBps_step": round(ls.bytes_per_step / (ms_f * 1e-3) / 1e9, 1),
                                          "unfused_ms_per_step": round(ms_plain, 5)}
    del ls
    torch.cuda.empty_cache()

    if not args.quick:
        iters = max(20, args.steps // 2)
        # 2x8 GEMV on the 7B block at batch 1, 4, 16
        for b in (1, 4, 16):
            ls2 = LayerSet(torch, "2x8", BLOCK_7B, b, sets_needed(BLOCK_7B, b), seed=1)
            if b == 1:
                spot_check(torch, E, ls2)
            ms2, sh2 = time_gemv(torch, E, ls2, iters, 5)
            ms2f = time_fused_block(torch, E, ls2, iters, 5)
            fused[f"2x8_b{b}"] = {"ms_per_step": round(ms2f, 5),
                                  "us_per_layer": round(ms2f * 1e3 / len(BLOCK_7B), 3),
                                  "GBps_step": round(ls2.bytes_per_step / (ms2f * 1e-3) / 1e9, 1),
                                  "unfused_ms_per_step": round(ms2, 5)}
            k2 = sum(sh2[sh] for sh in BLOCK_7B)
            breakdown[f"gemv_2x8_b{b}_7b_block"] = {
                "us_per_layer": round(k2 / len(BLOCK_7B), 3),
                "GBps_kernel": round(ls2.bytes_per_step / (k2 * 1e-6) / 1e9, 1),
                "GBps_step": round(ls2.bytes_per_step / (ms2 * 1e-3) / 1e9, 1),
                "per_shape": {f"{o}x{i}": {"us": round(us, 3),
                                           "GBps": round(gemv_bytes(o, i, b) / (us * 1e-6) / 1e9, 1)}
                              for (o, i), us in sh2.items()}}
            del ls2
            torch.cuda.empty_cache()
        # 70B layers, 1x16, batch 1
        r70 = {}
        for shape in SHAPES_70B:
            ls3 = LayerSet(torch, "1x16", (shape,), 1, sets_needed((shape,), 1, cap=16), seed=2)
            ls3.pack_lists(torch, E)
            _, sh3 = time_gemv(torch, E, ls3, iters, 5, lists=True)
            _, sh3p = time_gemv(torch, E, ls3, iters, 5)
            k3, k3p = sh3[shape], sh3p[shape]
            r70[f"{shape[0]}x{shape[1]}"] = {
                "us": round(k3, 3), "GBps": round(ls3.bytes_per_step / (k3 * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * ls3.bytes_per_step / (k3 * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                "stored_layout_us": round(k3p, 3),
                "stored_layout_GBps": round(ls3.bytes_per_step / (k3p * 1e-6) / 1e9, 1)}
            del ls3
            torch.cuda.empty_cache()
        t70 = sum(v["us"] for v in r70.values())
        b70 = sum(gemv_bytes(o, i, 1) for o, i in SHAPES_70B)
        r70["aggregate"] = {"what": "sum of bytes over sum of per-layer times, the four 70B shapes once each",
                            "us": round(t70, 3), "GBps": round(b70 / (t70 * 1e-6) / 1e9, 1),
                            "pct_hbm_peak": round(100 * b70 / (t70 * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        breakdown["gemv_1x16_b1_70b"] = r70
        # 70B layers, 2x8, batch 1: each shape alone, their aggregate, and a 70B block
        # step with q,k,v and gate,up fused (the streaming kernel's large layers)
        r70b = {}
        for shape in SHAPES_70B:
            ls4 = LayerSet(torch, "2x8", (shape,), 1, sets_needed((shape,), 1, cap=16), seed=4)
            _, sh4 = time_gemv(torch, E, ls4, iters, 5)
            k4 = sh4[shape]
            r70b[f"{shape[0]}x{shape[1]}"] = {
                "us": round(k4, 3), "GBps": round(ls4.bytes_per_step / (k4 * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * ls4.bytes_per_step / (k4 * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
            del ls4
            torch.cuda.empty_cache()
        t70b = sum(v["us"] for v in r70b.values())
        r70b["aggregate"] = {"what": "sum of bytes over sum of per-layer times, the four 70B shapes once each",
                             "us": round(t70b, 3), "GBps": round(b70 / (t70b * 1e-6) / 1e9, 1),
                             "pct_hbm_peak": round(100 * b70 / (t70b * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        ls5 = LayerSet(torch, "2x8", BLOCK_70B, 1, sets_needed(BLOCK_70B, 1, cap=8), seed=5)
        spot_check(torch, E, ls5)
        ms5 = time_fused_block(torch, E, ls5, max(10, iters // 2), 3)
        r70b["block_fused"] = {"what": "one 70B block per step: q,k,v fused | o | gate,up fused | down",
                               "ms_per_step": round(ms5, 5),
                               "GBps_step": round(ls5.bytes_per_step / (ms5 * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * ls5.bytes_per_step / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del ls5
        torch.cuda.empty_cache()
        breakdown["gemv_2x8_b1_70b"] = r70b
        breakdown["gemv_fused_7b_block"] = fused
        # prefill GEMM, 2048 tokens
        gen = torch.Generator(device="cuda")
        gen.manual_seed(3)
        gm = {}
        for scheme in ("2x8", "1x16"):
            cb = make_codebooks(torch, scheme, gen)
            for out, n_in in SHAPES_7B:
                codes = make_codes(torch, scheme, out, n_in, gen)
                s = make_scales(torch, out, gen)
                x = make_x(torch, 2048, n_in, gen)
                y = torch.empty((2048, out), dtype=torch.float16, device="cuda")
                us = time_calls(torch, lambda i: E.aqlm_linear_gemm(codes, cb, s, x, y), 10, 2)
                tf = 2.0 * 2048 * out * n_in / (us * 1e-6) / 1e12
                # two passes: the weights decoded once into a workspace, then the dense product
                M, B, g, _ = SCHEMES[scheme]
                ws = torch.empty((E.gemm_dequant_workspace_bytes(M, B, g, out, n_in),), dtype=torch.uint8,
                                 device="cuda")
                us2 = time_calls(torch, lambda i: E.aqlm_linear_gemm_dequant(codes, cb, s, x, y, ws), 10, 2)
                w16 = ws.view(torch.float16).view(out, n_in)
                usd = time_calls(torch, lambda i: E.aqlm_linear_decode(codes, cb, s, w16), 10, 2)
                tf2 = 2.0 * 2048 * out * n_in / (us2 * 1e-6) / 1e12
                gm[f"{scheme}_{out}x{n_in}"] = {"us": round(us, 1), "TFLOPs": round(tf, 1),
                                                "frac_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                                "two_pass_us": round(us2, 1),
                                                "two_pass_frac_mfma_peak": round(tf2 / MFMA_F16_PEAK_TFLOPS, 4),
                                                "two_pass_decode_us": round(usd, 1),
                                                "dense_product_frac_mfma_peak": round(
                                                    2.0 * 2048 * out * n_in / ((us2 - usd) * 1e-6) / 1e12
                                                    / MFMA_F16_PEAK_TFLOPS, 4)}
                del codes, s, x, y, ws, w16
            torch.cuda.empty_cache()
        breakdown["gemm_prefill_2048"] = gm
        # standalone decode, 4096x4096
        dc = {}
        for scheme in ("2x8", "1x16"):
            cb = make_codebooks(torch, scheme, gen)
            codes = make_codes(torch, scheme, 4096, 4096, gen)
            s = make_scales(torch, 4096, gen)
            w = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
            us = time_calls(torch, lambda i: E.aqlm_linear_decode(codes, cb, s, w), 20, 3)
            nbytes = 4096 * 4096 // 4 + 2 * 4096 + 2 * 4096 * 4096
            dc[f"{scheme}_4096x4096"] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        breakdown["decode"] = dc
        # generic schemes (the pages' other 2-bit pairs at B = 8), 4096x4096
        gs = {}
        for M, B, g in GENERIC_2BIT:
            cbg, codes = make_generic(torch, M, B, g, 4096, 4096, gen)
            s = make_scales(torch, 4096, gen)
            w = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
            x1 = make_x(torch, 1, 4096, gen)
            y1 = torch.empty((1, 4096), dtype=torch.float16, device="cuda")
            x16 = make_x(torch, 16, 4096, gen)
            y16 = torch.empty((16, 4096), dtype=torch.float16, device="cuda")
            x2 = make_x(torch, 2048, 4096, gen)
            y2 = torch.empty((2048, 4096), dtype=torch.float16, device="cuda")
            us_d = time_calls(torch, lambda i: E.aqlm_linear_decode(codes, cbg, s, w), 20, 3)
            # GEMV: 64 code sets (270 MB) in turn, so that no set is still in the last-level cache
            cset = [codes] + [make_generic(torch, M, B, g, 4096, 4096, gen)[1] for _ in range(63)]
            us_v = time_calls(torch, lambda i: E.aqlm_linear_gemv(cset[i % 64], cbg, s, x1, y1), 128, 3)
            us_v16 = time_calls(torch, lambda i: E.aqlm_linear_gemv(cset[i % 64], cbg, s, x16, y16), 128, 3)
            del cset
            us_m = time_calls(torch, lambda i: E.aqlm_linear_gemm(codes, cbg, s, x2, y2), 5, 1)
            wsg = torch.empty((E.gemm_dequant_workspace_bytes(M, B, g, 4096, 4096),), dtype=torch.uint8,
                              device="cuda")
            us_m2 = time_calls(torch, lambda i: E.aqlm_linear_gemm_dequant(codes, cbg, s, x2, y2, wsg), 5, 1)
            nb = generic_gemv_bytes(M, B, g, 4096, 4096, 1)
            dbytes = nb - 2 * 4096 - 2 * 4096 + 2 * 4096 * 4096
            gs[f"{M}x{B}g{g}_4096x4096"] = {
                "decode_us": round(us_d, 2), "decode_GBps": round(dbytes / (us_d * 1e-6) / 1e9, 1),
                "gemv_b1_us": round(us_v, 2), "gemv_b1_GBps": round(nb / (us_v * 1e-6) / 1e9, 1),
                "gemv_b16_us": round(us_v16, 2),
                "gemv_b16_GBps": round(generic_gemv_bytes(M, B, g, 4096, 4096, 16) / (us_v16 * 1e-6) / 1e9, 1),
                "gemm_2048_us": round(us_m, 1),
                "gemm_2048_frac_mfma_peak": round(2.0 * 2048 * 4096 * 4096 / (us_m * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                "gemm_2048_two_pass_us": round(us_m2, 1),
                "gemm_2048_two_pass_frac_mfma_peak": round(
                    2.0 * 2048 * 4096 * 4096 / (us_m2 * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
            del cbg, codes, s, w, x1, y1, x16, y16, x2, y2, wsg
            torch.cuda.empty_cache()
        breakdown["generic_schemes"] = gs
        # greedy residual encoder and residual k-means (3 unfused fp32 ops per codeword entry compared)
        en = {}
        for (M, B, g, out, n_in, iters) in ((2, 8, 8, 4096, 4096, 0), (2, 8, 8, 4096, 4096, 10),
                                            (1, 16, 8, 1024, 4096, 0)):
            w = (torch.randn((out, n_in), generator=gen, device="cuda") * 0.05).half()
            s = ((torch.rand(out, generator=gen, device="cuda") + 0.5) * 0.05).half()
            cbg = torch.randn((M, 1 << B, g), generator=gen, device="cuda").half()
            n_grp = out * n_in // g
            if iters == 0:
                us = time_calls(torch, lambda i: E.aqlm_encode_greedy(w, s, cbg), 3, 1)
                ops = 3.0 * n_grp * (1 << B) * g * M
                en[f"greedy_{M}x{B}g{g}_{out}x{n_in}"] = {
                    "us": round(us, 1), "Tops": round(ops / (us * 1e-6) / 1e12, 2),
                    "frac_valu_peak": round(ops / (us * 1e-6) / 1e12 / VALU_F32_PEAK_TOPS, 4)}
            else:
                seeds = torch.randint(0, n_grp, (M, 1 << B), generator=gen, device="cuda", dtype=torch.int64)
                ws = torch.empty(E.kmeans_workspace_bytes(M, B, g), dtype=torch.uint8, device="cuda")
                us = time_calls(torch, lambda i: E.aqlm_kmeans_init(w, s, seeds, B, g, iters, workspace=ws), 2, 1)
                ops = 3.0 * n_grp * (1 << B) * g * M * (iters + 1)
                en[f"kmeans_{M}x{B}g{g}_{out}x{n_in}_iters{iters}"] = {
                    "us": round(us, 1), "Tops": round(ops / (us * 1e-6) / 1e12, 2),
                    "frac_valu_peak": round(ops / (us * 1e-6) / 1e12 / VALU_F32_PEAK_TOPS, 4)}
            del w, s, cbg
            torch.cuda.empty_cache()
        breakdown["encode"] = en
        # fp16 comparator (torch.matmul on dense fp16 weights: the vendor BLAS), the
        # denominator of the "speedup vs FP16" figures the AQLM pages quote.
        cmp16 = {}
        aq1 = {k: v["us"] for k, v in per_shape.items()}
        aq1p = {k: v["us"] for k, v in breakdown["gemv_1x16_b1_7b_stored_layout"]["per_shape"].items()}
        aq2 = breakdown["gemv_2x8_b1_7b_block"]["per_shape"]
        for out, n_in in SHAPES_7B:
            n = max(2, min(32, -(-LLC_BYTES * 2 // (2 * out * n_in))))
            ws16 = [torch.randn((out, n_in), generator=gen, device="cuda", dtype=torch.float32).half()
                    for _ in range(n)]
            xv = make_x(torch, 1, n_in, gen)
            us16 = time_calls(torch, lambda i: torch.matmul(xv, ws16[i % n].t()), 4 * n, 2)
            key = f"{out}x{n_in}"
            cmp16[key] = {"fp16_us": round(us16, 3),
                          "speedup_1x16": round(us16 / aq1[key], 3),
                          "speedup_1x16_stored_layout": round(us16 / aq1p[key], 3),
                          "speedup_2x8": round(us16 / aq2[key]["us"], 3)}
            del ws16
            torch.cuda.empty_cache()
        breakdown["gemv_b1_vs_fp16"] = cmp16

    if args.copy_probe:
        src = torch.empty(32 << 20, dtype=torch.float16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None if (args.quick or args.no_cpu) else cpu_baseline()

    rec = {
        "metric": "AQLM 2-bit linear us/layer + achieved HBM GB/s (% peak), 7B/70B shapes",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-2-7B decoder-block projections (q,k,v,o 4096x4096; gate,up 11008x4096; "
                        "down 4096x11008) as AQLM 1x16 g8 decode GEMV, batch 1",
            "scheme": "1x16", "group": 8, "batch": 1, "layers_per_step": len(BLOCK_7B),
            "codes_layout": "slice lists (aqlm_lists_pack once per layer at load, outside the timed region; "
                            "the stored layout's figures are under breakdown)",
            "entry_bytes_per_step": int(entry_bytes_step),
            "served_bits_per_weight": round(8.0 * entry_bytes_step / sum(o * i for o, i in BLOCK_7B), 3),
            "stored_layout_GBps": (None if args.quick else
                                   breakdown["gemv_1x16_b1_7b_stored_layout"]["GBps_step"]),
            "rotated_buffer_sets": n_sets, "parallelism": "single GPU",
            "us_per_layer": round(ms_step * 1e3 / len(BLOCK_7B), 3),
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "pct_measured_copy_bw": round(100 * value / copy_gbps, 2),
            "effective_weight_GBps": round(sum(2 * o * i for o, i in BLOCK_7B) / (ms_step * 1e-3) / 1e9, 1),
            "spot_check_rel_l2": worst,
            "device": dev_name,
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": "gemv_lists_kernel + lists_reduce_kernel (one aqlm_linear_gemv_lists call)",
                     "kernel_us_per_step": round(kern_us_step, 3),
                     "method": "per-shape mean duration of back-to-back launches replayed from a HIP graph"},
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
