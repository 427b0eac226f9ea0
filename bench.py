#!/usr/bin/env python3
"""Benchmark of the dense linear-layer GEMM C = A * B^T on one MI355X.

Default workload: bf16 M = N = K = 4096 (A, B ~ N(0, 0.02^2), B stored [N, K]
and preshuffled once).  A step is one GEMM call through the C ABI with the
tile chosen by select_tile; the preshuffle is a once-per-weight cost timed
separately.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Measurement:
  * W untimed warm-up calls, then exactly K calls bracketed by
    torch.cuda.synchronize() on both sides, timed with HIP events on the
    stream the kernels run on (torch's current stream); the calls run back
    to back, so total time / K is the average launch duration.  The K calls
    are replayed from one HIP graph, enqueued right behind the W warm-up
    calls, so that the start event is reached with the device busy.
  * `sustained`: the same graph replayed back to back for --soak seconds,
    each replay timed by its own events, the shader clock and board power
    sampled inside the timed half; `roofline.frac_at_sustained_clock` rates
    that figure against the MFMA peak at the sampled clock.  With --soak > 0
    the W warm-ups and the K timed calls run once from idle (reported as
    `sustained.from_idle_ms_per_step`: the clock is still ramping up) and
    again right after the sustained replay; `value` is that second run, the
    board's loaded power state.
  * The K calls rotate over enough copies of (A, Bs, C) to exceed twice the
    256 MB Infinity Cache, so every call reads its operands from HBM.
  * `roofline`: algorithmic flops (2MNK, "GEMM Optimization Guide" page,
    section 8.1) or bytes per launch over the average kernel duration,
    against MI355X's published dense peak or HBM bandwidth.
  * `cpu_baseline`: the oracle (plain C fp64 triple loop) on a bounded sample
    of the same workload -- whole rows of C -- timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

# --------------------------------------------------------------- formulas
# Dense peaks and HBM bandwidth of one MI355X (AMD's published figures; dense,
# no sparsity): 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20
CUS = 256
# split-K / stream-K: the workspace the bench hands the library (the selector
# weighs split-K tiles whose fp32 partials fit, the launch plan stream-K), and
# the slice counts a sweep tries
WORKSPACE_MIB = 128
SPLITS = (2, 3, 4, 6, 8, 12, 16)
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
# The device code whose hash identifies "the kernel" a traffic measurement
# belongs to: a measurement taken on other sources is not reported.
KERNEL_SOURCES = ["device.hpp", "kernels.hpp", "tiled_inst.hip",
                  "skinny.hip"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_gemm_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, tile_name: str):
    """HBM bytes per launch measured by rocprofv3 counters for this workload
    (profiles/traffic_<workload>.json, written by --traffic-summary), or None
    if absent or taken on another rung or other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("tile") != tile_name or t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def flops(M: int, N: int, K: int) -> float:
    """2*M*N*K: each multiply-add is two flops ("GEMM Optimization Guide"
    page, section 8.1)."""
    return 2.0 * M * N * K


def alg_bytes(M: int, N: int, K: int, dtype: str, scales: str = "per_tensor") -> float:
    """Algorithmic HBM bytes: every operand read once and C written once.

    bf16: 2*(M*K + N*K + M*N) (the 16-bit operand/output reading of the
    FLOPS/Byte column on the TraceLens GEMM analysis page).  fp8: the
    "GEMM Optimization Guide" page, section 8.2 (1-byte A and B, bf16 C) with
    the scales as stored: two fp32 per-tensor scales (8 bytes) here, or
    (M + N) fp32 per-token scales as on that page."""
    if dtype == "bf16":
        return 2.0 * (M * K + N * K + M * N)
    if dtype == "fp8":
        sc = 8.0 if scales == "per_tensor" else 4.0 * (M + N)
        return 1.0 * M * K + 1.0 * N * K + 2.0 * M * N + sc
    raise ValueError(dtype)


def tflops_at(M: int, N: int, K: int, us: float) -> float:
    return flops(M, N, K) / (us * 1e-6) / 1e12


def roofline_us(M: int, N: int, K: int, dtype: str) -> float:
    """Lower bound on time: max of the MFMA time and the HBM time."""
    t_c = flops(M, N, K) / (PEAK_TFLOPS[dtype] * 1e12)
    t_m = alg_bytes(M, N, K, dtype) / (PEAK_HBM_GBPS * 1e9)
    return max(t_c, t_m) * 1e6


# (M, N, K, dtype, dist A, sigma A, dist B, sigma B, seed config)
WORKLOADS = {
    "bf16_4096cube": (4096, 4096, 4096, "bf16", "normal", 0.02, "normal", 0.02, 2),
    "bf16_llama_prefill": (597, 11008, 4096, "bf16", "normal", 1.0, "normal", 0.02, 3),
    "bf16_llama_decode": (1, 11008, 4096, "bf16", "normal", 1.0, "normal", 0.02, 3),
    "bf16_8x4096": (8, 4096, 4096, "bf16", "normal", 1.0, "normal", 1.0, 42),
    "bf16_48x4096": (48, 4096, 4096, "bf16", "normal", 1.0, "normal", 1.0, 43),
    "bf16_3402x4096x1024": (3402, 4096, 1024, "bf16", "normal", 1.0, "normal", 1.0, 44),
    "bf16_lmhead_1024x50257x512": (1024, 50257, 512, "bf16", "normal", 1.0, "normal", 1.0, 45),
    "bf16_2048x11007x1024": (2048, 11007, 1024, "bf16", "normal", 1.0, "normal", 1.0, 46),
    "bf16_4095x4095x1024": (4095, 4095, 1024, "bf16", "normal", 1.0, "normal", 1.0, 47),
    "bf16_528x528x1024": (528, 528, 1024, "bf16", "normal", 1.0, "normal", 1.0, 48),
    # one GPU's share of the LLaMA-2-7B MLP under 8-way tensor parallelism:
    # column-parallel up/gate (N = 11008 / 8) at prefill and decode, and the
    # row-parallel down projection (K = 11008 / 8)
    "bf16_tp8_up_597x1376x4096": (597, 1376, 4096, "bf16", "normal", 1.0, "normal", 0.02, 61),
    "bf16_tp8_decode_1x1376x4096": (1, 1376, 4096, "bf16", "normal", 1.0, "normal", 0.02, 62),
    "bf16_tp8_down_597x4096x1376": (597, 4096, 1376, "bf16", "normal", 1.0, "normal", 0.02, 63),
    # GPT-3-XL training GEMMs (batch 5 x 2048 tokens, d_model 2048, d_ff 8192):
    # forward up projection, and the backward dX (K = d_ff) and dW (K = tokens)
    "bf16_gpt3xl_fwd_10240x8192x2048": (10240, 8192, 2048, "bf16", "normal", 1.0, "normal", 0.02, 81),
    "bf16_gpt3xl_dgrad_10240x2048x8192": (10240, 2048, 8192, "bf16", "normal", 1.0, "normal", 0.02, 82),
    "bf16_gpt3xl_wgrad_8192x2048x10240": (8192, 2048, 10240, "bf16", "normal", 1.0, "normal", 1.0, 83),
    "fp8_4096cube": (4096, 4096, 4096, "fp8", "normal", 1.0, "normal", 1.0, 5),
    "fp8_tp8_up_597x1376x4096": (597, 1376, 4096, "fp8", "normal", 1.0, "normal", 1.0, 64),
    "fp8_32x4096": (32, 4096, 4096, "fp8", "normal", 1.0, "normal", 1.0, 51),
    # more small-M shapes for the selector's calibration of the skinny rungs
    "bf16_1x4096x4096": (1, 4096, 4096, "bf16", "normal", 1.0, "normal", 0.02, 71),
    "bf16_2x8192x8192": (2, 8192, 8192, "bf16", "normal", 1.0, "normal", 0.02, 72),
    "bf16_16x4096x4096": (16, 4096, 4096, "bf16", "normal", 1.0, "normal", 0.02, 73),
    "bf16_32x11008x4096": (32, 11008, 4096, "bf16", "normal", 1.0, "normal", 0.02, 74),
    "bf16_64x4096x4096": (64, 4096, 4096, "bf16", "normal", 1.0, "normal", 0.02, 75),
    "bf16_1x28672x8192": (1, 28672, 8192, "bf16", "normal", 1.0, "normal", 0.02, 76),
    "bf16_12x2048x8192": (12, 2048, 8192, "bf16", "normal", 1.0, "normal", 0.02, 77),
    "fp8_8x11008x4096": (8, 11008, 4096, "fp8", "normal", 1.0, "normal", 1.0, 78),
    "bf16_16x11008x4096": (16, 11008, 4096, "bf16", "normal", 1.0, "normal", 0.02, 86),
    "bf16_16x8192x8192": (16, 8192, 8192, "bf16", "normal", 1.0, "normal", 0.02, 87),
    "fp8_597x11008x4096": (597, 11008, 4096, "fp8", "normal", 1.0, "normal", 1.0, 79),
    "fp8_2048x8192x2048": (2048, 8192, 2048, "fp8", "normal", 1.0, "normal", 1.0, 80),
    "fp8_8192x4096x4096": (8192, 4096, 4096, "fp8", "normal", 1.0, "normal", 1.0, 85),
    # held out of the selector's calibration (their sweeps are kept apart, in
    # calibration/mi355x_holdout.jsonl): how well it prices shapes it never saw
    "bf16_256x4096x4096": (256, 4096, 4096, "bf16", "normal", 1.0, "normal", 0.02, 91),
    "bf16_2048x4096x4096": (2048, 4096, 4096, "bf16", "normal", 1.0, "normal", 0.02, 92),
    "bf16_1024x14336x4096": (1024, 14336, 4096, "bf16", "normal", 1.0, "normal", 0.02, 93),
    "bf16_1024x4096x14336": (1024, 4096, 14336, "bf16", "normal", 1.0, "normal", 0.02, 94),
    "bf16_16x14336x4096": (16, 14336, 4096, "bf16", "normal", 1.0, "normal", 0.02, 95),
    "bf16_4x4096x11008": (4, 4096, 11008, "bf16", "normal", 1.0, "normal", 0.02, 96),
    "bf16_8192x1024x1024": (8192, 1024, 1024, "bf16", "normal", 1.0, "normal", 0.02, 97),
    "bf16_333x5000x2048": (333, 5000, 2048, "bf16", "normal", 1.0, "normal", 0.02, 98),
    "fp8_1024x14336x4096": (1024, 14336, 4096, "fp8", "normal", 1.0, "normal", 1.0, 99),
}
HEADLINE = "bf16_4096cube"
DECODE = "bf16_llama_decode"


def bound_of(M, N, K, dtype) -> str:
    t_c = flops(M, N, K) / (PEAK_TFLOPS[dtype] * 1e12)
    t_m = alg_bytes(M, N, K, dtype) / (PEAK_HBM_GBPS * 1e9)
    return "mfma" if t_c >= t_m else "hbm"


# ------------------------------------------------------------- GPU timing
def make_inputs(name: str):
    import numpy as np
    import datagen
    M, N, K, dt, da, sa, db, sb, cfg = WORKLOADS[name]
    if dt == "bf16":
        A, B = datagen.make_bf16_pair(M, N, K, da, db, cfg, sa, sb)
        return A, B, 1.0, 1.0
    A, B, s_a, s_b = datagen.make_e4m3_pair(M, N, K, cfg)
    return A, B, s_a, s_b


def cold_copies(per_set: float) -> int:
    """Operand sets whose total exceeds twice the Infinity Cache, so that a
    rotation over them reads every operand from HBM (small shards included:
    each set is touched again only after the others have passed through)."""
    return max(1, int(2 * MALL_BYTES // per_set) + 1)


def gpu_setup(name: str, copies: int):
    import numpy as np
    import torch
    import dense_gemm_linear_amd as dg
    M, N, K, dt = WORKLOADS[name][:4]
    A, B, s_a, s_b = make_inputs(name)
    if dt == "bf16":
        Ad = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
        Bd = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        Ad = torch.from_numpy(A).cuda()
        Bd = torch.from_numpy(B).cuda()
    # preshuffle, timed on its own
    Bs0 = dg.shuffle_b(Bd, dtype=dt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reps = 5
    for _ in range(reps):
        dg.shuffle_b(Bd, dtype=dt, out=Bs0)
    e1.record()
    torch.cuda.synchronize()
    shuffle_us = e0.elapsed_time(e1) * 1e3 / reps
    sets = []
    for i in range(copies):
        a = Ad if i == 0 else Ad.clone()
        bs = Bs0 if i == 0 else Bs0.clone()
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        sets.append((a, bs, c))
    scales = (torch.tensor([s_a], dtype=torch.float32, device="cuda"),
              torch.tensor([s_b], dtype=torch.float32, device="cuda"))
    del Bd
    return sets, scales, shuffle_us


def parse_tile(spec: str | None):
    """'tiled:256x128', 'tiled:256x256w8', 'ab:256x256w8a32s4k32' or 'skinny:16x32'
    -> Tile (suffixes: aR = R x R MFMA atom, sN = N stages, kE = E K elements per
    stage); None -> select_tile."""
    if spec is None:
        return None
    import re
    import dense_gemm_linear_amd as dg
    kind, dims = spec.split(":")
    atom, stages, tile_k = 16, 0, 0
    stream_k = dims.endswith("streamk")
    if stream_k:
        dims = dims[:-len("streamk")]
    m = re.fullmatch(r"(\d+x\d+(?:w\d+)?)(?:a(\d+))?(?:s(\d+))?(?:k(\d+))?(?:sk(\d+))?", dims)
    if not m:
        raise ValueError(f"bad tile spec {spec!r}")
    dims = m.group(1)
    atom = int(m.group(2) or 16)
    stages = int(m.group(3) or 0)
    tile_k = int(m.group(4) or 0)
    k_split = int(m.group(5) or 1)
    waves = 4
    if "w" in dims:
        dims, w = dims.split("w")
        waves = int(w)
    tm, tn = (int(x) for x in dims.split("x"))
    if kind == "tiled":
        t = dg.tiled(tm, tn, waves, atom, stages, tile_k, k_split)
        return dg.with_stream_k(t) if stream_k else t
    if kind == "ab":
        t = dg.tiled_ab(tm, tn, waves, atom, stages, tile_k, k_split)
        return dg.with_stream_k(t) if stream_k else t
    if kind == "pp":
        return dg.tiled_pp(tm, tn, atom, stages, tile_k, k_split)
    return dg.skinny(tm, tn, waves)


def run_timed(name: str, steps: int, warmup: int, copies: int | None = None, per_launch=True,
              tile=None, setup=None, soak: float = 0.0, workspace=None, graph: bool = False):
    """W eager warm-up calls, then K timed calls with one HIP event pair
    around them on the kernels' stream.  graph=True captures the K calls in
    one HIP graph and times its replay (no host submission gaps between
    short kernels); otherwise they are issued eagerly, optionally with an
    event pair around each (per_launch)."""
    import torch
    import dense_gemm_linear_amd as dg
    M, N, K, dt = WORKLOADS[name][:4]
    if copies is None:
        copies = cold_copies(alg_bytes(M, N, K, dt))
    if setup is None:
        setup = gpu_setup(name, copies)
    sets, (s_a, s_b), shuffle_us = setup
    copies = len(sets)
    forced = tile
    ws_bytes = 0 if workspace is None else workspace.numel()
    if tile is None:   # the library's launch plan (its first launch)
        tile = dg.plan(M, N, K, dt, CUS, ws_bytes)[0]

    def call(i):
        a, bs, c = sets[i % copies]
        if dt == "bf16":
            dg.gemm_bf16(a, bs, N, out=c, tile=forced, workspace=workspace)
        else:
            dg.gemm_fp8_scaled(a, bs, N, s_a, s_b, out=c, tile=forced, workspace=workspace)

    if graph:
        # One call ahead of the capture (lazy initialisation of the code
        # object), then the K timed calls captured in one HIP graph.
        call(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    call(warmup + i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # The W warm-up calls are enqueued right ahead of the timed replay,
        # with no synchronisation between: the GPU runs them while the host
        # submits the replay, so the start event is reached with the device
        # busy, and the K timed calls follow back to back.  (A spin kernel
        # in their place let the shader clock sink before the timed calls:
        # an isolated launch after an idle gap ran at 1.2-1.4 GHz.)
        def timed_replay():
            wall0 = time.perf_counter()
            for i in range(warmup):
                call(i)
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1), time.perf_counter() - wall0

        total_ms, wall = timed_replay()
        sustained = None
        if soak > 0:
            # The board starts from idle: its shader clock ramps up over the
            # first milliseconds, so K steps timed right away mix the ramp
            # with the loaded state.  After the sustained replay (about
            # `soak` seconds, timed by its own events) the W warm-ups and the
            # K timed steps are run once more: the reported K-step time is
            # the loaded power state's, and the first one is kept as context.
            sustained = sustained_with_clock(g, steps, soak)
            sustained["from_idle_ms_per_step"] = round(total_ms / steps, 5)
            total_ms, wall = timed_replay()
        del g
        return {"total_ms": total_ms, "wall_s": wall, "kernel_us": [], "tile": tile,
                "shuffle_us": shuffle_us, "copies": copies, "sustained": sustained}
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)] if per_launch else []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        if per_launch:
            ev[i][0].record(stream)
        call(i)
        if per_launch:
            ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    kern_us = [s.elapsed_time(e) * 1e3 for s, e in ev] if per_launch else []
    return {
        "total_ms": total_ms, "wall_s": wall, "kernel_us": kern_us, "tile": tile,
        "shuffle_us": shuffle_us, "copies": copies, "sustained": None,
    }


def sustained_with_clock(g, steps: int, seconds: float):
    """sustained_replay with clock / power samples taken inside the timed
    second half (replays stay queued while the samples are read)."""
    import torch
    out = {"samples": []}
    t_start = time.perf_counter()
    next_sample = 0.0
    evs = []
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        evs.append((e0, e1))
        now = time.perf_counter() - t_start
        if len(evs) >= 3:
            evs[-3][1].synchronize()
        if now >= seconds / 2 and now >= next_sample and "error" not in out:
            next_sample = now + 0.05      # every 50 ms: the queries take host time
            try:
                out["samples"].append((torch.cuda.clock_rate(), torch.cuda.power_draw()))
            except Exception as e:  # noqa: BLE001 - any query failure means "unavailable"
                out["error"] = f"{type(e).__name__}: {e}"
        if now >= seconds:
            break
    torch.cuda.synchronize()
    half = len(evs) // 2
    per_call = sorted(a.elapsed_time(b) * 1e3 / steps for a, b in evs[half:])
    mhz = [c for c, _ in out["samples"]]
    watts = [p / 1000.0 if p > 20000 else float(p) for _, p in out["samples"]]
    return {"per_call_us": round(per_call[len(per_call) // 2], 3), "replays": len(evs),
            "timed_replays": len(evs) - half, "seconds": round(time.perf_counter() - t_start, 3),
            "gfx_mhz_mean": round(sum(mhz) / len(mhz), 1) if mhz else None,
            "gfx_mhz_min_max": [min(mhz), max(mhz)] if mhz else None,
            "power_w_mean": round(sum(watts) / len(watts), 1) if watts else None,
            "clock_samples": len(mhz), **({"error": out["error"]} if "error" in out else {})}


def hold_stream(stream=None):
    """Enqueue about a millisecond of device work (a bounded spin kernel) on
    the stream, ahead of a timed graph replay: the GPU then reaches the start
    event only after the host has submitted the graph, so the event pair times
    the kernels back to back and not the host's submission of the graph."""
    import torch
    with torch.cuda.stream(stream or torch.cuda.current_stream()):
        torch.cuda._sleep(2_000_000)


def time_graph(call, reps: int, trials: int = 1) -> float:
    """Per-launch time of `call` (launches only: no allocation, no memset,
    the kernels write every output element themselves) from R calls captured
    in one HIP graph: the median over `trials` graphs of replay time / R.
    Each trial has a graph of its own over the next R operand sets (call(i)
    takes set i mod the number of copies), replayed once, so a small
    workload's trials do not re-read the sets the previous one left in the
    Infinity Cache.  Kernels shorter than a Python launch are timed without
    the host's submission gaps this way."""
    import torch
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for t in range(trials):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(reps):
                    call(3 + t * reps + i)
        graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    per = []
    for g in graphs:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_stream()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) * 1e3 / reps)
    del graphs
    return sorted(per)[len(per) // 2]


def gemm_call(name: str, sets, scales, tile=None, workspace=None):
    """call(i): one GEMM of the workload on operand set i mod len(sets)."""
    import dense_gemm_linear_amd as dg
    N, dt = WORKLOADS[name][1], WORKLOADS[name][3]
    s_a, s_b = scales

    def call(i):
        a, bs, c = sets[i % len(sets)]
        if dt == "bf16":
            dg.gemm_bf16(a, bs, N, out=c, tile=tile, workspace=workspace)
        else:
            dg.gemm_fp8_scaled(a, bs, N, s_a, s_b, out=c, tile=tile, workspace=workspace)
    return call


def epilogue_compare(name: str, spec: str, reps: int, ws_mib: int) -> int:
    """The fused epilogue against the same work done by a caller without it:
    the plain GEMM, then the epilogue as torch elementwise ops on C.  Both
    graph-timed; one JSON line.  spec: comma-separated parts of scale_m,
    scale_n, bias, mul and at most one activation (relu, silu, gelu,
    gelu_tanh)."""
    import torch
    import dense_gemm_linear_amd as dg
    M, N, K, dt = WORKLOADS[name][:4]
    parts = [p for p in spec.split(",") if p]
    acts = [p for p in parts if p in dg.ACTIVATIONS and p != "none"]
    unknown = [p for p in parts if p not in ("scale_m", "scale_n", "bias", "mul") and p not in acts]
    if unknown or len(acts) > 1:
        print(f"bench.py: bad --epilogue {spec!r}", file=sys.stderr)
        return 2
    act = acts[0] if acts else None
    per_set = alg_bytes(M, N, K, dt) + (2 * M * N if "mul" in parts else 0)
    copies = cold_copies(per_set)
    sets, (s_a, s_b), _ = gpu_setup(name, copies)
    g = torch.Generator(device="cuda").manual_seed(7)
    kw = {}
    if "scale_m" in parts:
        kw["scale_m"] = torch.rand(M, device="cuda", generator=g) + 0.5
    if "scale_n" in parts:
        kw["scale_n"] = torch.rand(N, device="cuda", generator=g) + 0.5
    if "bias" in parts:
        kw["bias"] = torch.randn(N, device="cuda", generator=g).bfloat16()
    muls = [torch.randn(M, N, device="cuda", generator=g).bfloat16() for _ in range(copies)] \
        if "mul" in parts else None
    workspace = torch.empty(max(ws_mib << 20, 16), dtype=torch.uint8, device="cuda")
    torch_act = {"relu": torch.relu, "silu": torch.nn.functional.silu,
                 "gelu": torch.nn.functional.gelu, "gelu_erf": torch.nn.functional.gelu,
                 "gelu_tanh": lambda x: torch.nn.functional.gelu(x, approximate="tanh")}

    def gemm(i, **extra):
        a, bs, c = sets[i % copies]
        if dt == "bf16":
            dg.gemm_bf16(a, bs, N, out=c, workspace=workspace, **extra)
        else:
            dg.gemm_fp8_scaled(a, bs, N, s_a, s_b, out=c, workspace=workspace, **extra)
        return c

    def fused(i):
        extra = dict(kw)
        if muls is not None:
            extra["mul"] = muls[i % copies]
        gemm(i, activation=act, **extra)

    def unfused(i):
        c = gemm(i)
        y = c.float()
        if "scale_m" in kw:
            y = y * kw["scale_m"][:, None]
        if "scale_n" in kw:
            y = y * kw["scale_n"][None, :]
        if "bias" in kw:
            y = y + kw["bias"].float()[None, :]
        if act:
            y = torch_act[act](y)
        if muls is not None:
            y = y * muls[i % copies].float()
        c.copy_(y.bfloat16())

    t_plain = time_graph(lambda i: gemm(i), reps, trials=3)
    t_fused = time_graph(fused, reps, trials=3)
    t_unfused = time_graph(unfused, reps, trials=3)
    print(json.dumps({"epilogue": spec, "workload": name,
                      "tile": dg.select_tile(M, N, K, dt, workspace_bytes=workspace.numel()).name,
                      "plain_gemm_us": round(t_plain, 3), "fused_us": round(t_fused, 3),
                      "gemm_then_torch_epilogue_us": round(t_unfused, 3),
                      "timing": f"hipGraph of {reps} calls, median of 3 replays"}), flush=True)
    return 0


def backward_prep(reps: int) -> int:
    """The memory-bound steps the backward GEMMs add, at GPT-3-XL sizes,
    graph-timed: transpose_2d of dY [10240, 8192] (the A of dW), shuffle_b_t
    of W [8192, 2048] (the B of dX) and of X [10240, 2048] (the B of dW).
    Bytes = read + written."""
    import torch
    import dense_gemm_linear_amd as dg
    T, D, F = 10240, 2048, 8192
    g = torch.Generator(device="cuda").manual_seed(3)
    # (source, destination) pairs rotated cold, as for the GEMM workloads
    def pairs(shape, dst_of):
        n = cold_copies(2 * shape[0] * shape[1] * 2)
        src = torch.randn(*shape, device="cuda", generator=g).bfloat16()
        return [(src if i == 0 else src.clone(), dst_of()) for i in range(n)]
    dYs = pairs((T, F), lambda: torch.empty(F, T, dtype=torch.bfloat16, device="cuda"))
    Wss = pairs((F, D), lambda: torch.empty(dg.shuffle_b_bytes(D, F), dtype=torch.uint8, device="cuda"))
    Xss = pairs((T, D), lambda: torch.empty(dg.shuffle_b_bytes(D, T), dtype=torch.uint8, device="cuda"))
    out = {}
    for label, ps, fn in (
            ("transpose_dY_10240x8192", dYs, lambda s, d: dg.transpose(s, out=d)),
            ("shuffle_b_t_W_8192x2048", Wss, lambda s, d: dg.shuffle_b_t(s, out=d)),
            ("shuffle_b_t_X_10240x2048", Xss, lambda s, d: dg.shuffle_b_t(s, out=d))):
        nbytes = ps[0][0].numel() * 2 + ps[0][1].numel() * ps[0][1].element_size()
        us = time_graph(lambda i, ps=ps, fn=fn: fn(*ps[i % len(ps)]), reps, trials=3)
        out[label] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    print(json.dumps({"backward_prep": out, "timing": f"hipGraph of {reps} calls, median of 3, "
                                                   f"operands rotated cold"}),
          flush=True)
    return 0


def run_graph(name: str, reps: int, copies: int):
    """Decode-size kernels are shorter than a Python launch: time R launches
    captured in one HIP graph."""
    sets, scales, shuffle_us = gpu_setup(name, copies)
    return time_graph(gemm_call(name, sets, scales), reps), shuffle_us


def read_floor_us(nbytes: int, reps: int = 60) -> float:
    """Per-launch time of the library's streaming-read probe over nbytes of
    device memory, timed as the decode kernels are (a HIP graph of R launches
    over enough buffer copies to exceed twice the Infinity Cache): the floor
    under any kernel that reads those bytes once from HBM."""
    import torch
    import dense_gemm_linear_amd as dg
    nbytes = (nbytes + 15) // 16 * 16
    copies = cold_copies(nbytes)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i & 0xFF) for i in range(copies)]
    out = torch.empty(dg.READ_PROBE_SLOTS, dtype=torch.int32, device="cuda")
    us = time_graph(lambda i: dg.read_probe(bufs[i % copies], out=out), reps, trials=3)
    del bufs
    return us


def read_floor_report(names) -> int:
    """One JSON line per workload: the bytes it must read from HBM (its
    algorithmic bytes less C) and the streaming-read probe's time for them."""
    for name in names:
        M, N, K, dt = WORKLOADS[name][:4]
        e = 2 if dt == "bf16" else 1
        nbytes = (M + N) * K * e
        us = read_floor_us(nbytes)
        print(json.dumps({"read_floor": name, "bytes": nbytes, "probe_us": round(us, 3),
                          "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}), flush=True)
    return 0


def _safe(f):
    """f(), or the error's text: for context figures that must not cost the
    bench line if they fail."""
    try:
        return f()
    except Exception as e:  # noqa: BLE001
        return f"error: {type(e).__name__}: {e}"[:200]


def hipblaslt_same_box(name: str, steps: int, warmup: int, soak: float):
    """The same workload through torch's matmul (hipBLASLt on ROCm; fp8 via
    torch._scaled_mm with unit scales), timed exactly as the library's call:
    W warm-ups ahead of a graph replay of K calls over the same number of
    cold operand copies, then a sustained replay.  Context for the library's
    figure on the same box and in the same power state, not a baseline from
    the pages."""
    import torch
    M, N, K, dt = WORKLOADS[name][:4]
    e = 2 if dt == "bf16" else 1
    copies = cold_copies(alg_bytes(M, N, K, dt))
    g = torch.Generator(device="cuda").manual_seed(7)
    sets = []
    for _ in range(copies):
        a = torch.randn(M, K, device="cuda", generator=g)
        b = torch.randn(N, K, device="cuda", generator=g) * 0.02
        if dt == "bf16":
            sets.append((a.bfloat16(), b.bfloat16(), torch.empty(M, N, dtype=torch.bfloat16, device="cuda")))
        else:
            sets.append((a.to(torch.float8_e4m3fn), (b * 50).to(torch.float8_e4m3fn),
                         torch.empty(M, N, dtype=torch.bfloat16, device="cuda")))
    one = torch.ones((), device="cuda")

    def call(i):
        a, b, c = sets[i % copies]
        if dt == "bf16":
            torch.mm(a, b.t(), out=c)
        else:
            torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16, out=c)

    call(0)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(gr, stream=side):
            for i in range(steps):
                call(warmup + i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    sus = sustained_with_clock(gr, steps, soak) if soak > 0 else None
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        call(i)
    t0.record()
    gr.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    del gr
    out = {"us_per_call": round(us, 3), "TFLOPs": round(flops(M, N, K) / (us * 1e-6) / 1e12, 2)}
    if sus:
        out["sustained_us_per_call"] = sus["per_call_us"]
        out["sustained_gfx_mhz_mean"] = sus["gfx_mhz_mean"]
    out["timing"] = ("torch.mm / torch._scaled_mm (hipBLASLt), K calls replayed from one HIP graph "
                     "after the sustained replay, same operand rotation as the library's")
    return out


# ------------------------------------------------------------ CPU oracle
def cpu_baseline(name: str, budget_s: float = 20.0):
    """The oracle on whole rows of C of the same workload, scaled to TFLOP/s."""
    import numpy as np
    import oracle
    M, N, K, dt = WORKLOADS[name][:4]
    A, B, s_a, s_b = make_inputs(name)
    threads = min(16, os.cpu_count() or 1)
    rows = threads
    while True:
        t = time.perf_counter()
        if dt == "bf16":
            oracle.gemm_bf16(A[:rows], B, threads=threads)
        else:
            oracle.gemm_e4m3(A[:rows], B, s_a, s_b, threads=threads)
        el = time.perf_counter() - t
        if el >= budget_s / 2 or rows >= M:
            break
        rows = min(M, max(rows * 2, int(rows * budget_s / 2 / max(el, 1e-3))))
    val = flops(rows, N, K) / el / 1e12
    return {"value": val, "unit": "TFLOP/s", "cores": threads, "host_cpu_count": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{rows} whole rows of C ({rows}x{N}x{K}, {rows * N * K / 1e9:.2f} G multiply-adds, "
                      f"fp64 triple loop on {threads} threads) in {el:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode measurement")
    ap.add_argument("--copies", type=int, default=0,
                    help="operand sets rotated through the timed calls (0 = enough to exceed twice "
                         "the Infinity Cache, so operands come from HBM; 1 = hot cache)")
    ap.add_argument("--soak", type=float, default=1.5,
                    help="seconds of back-to-back replays of the timed graph after the timed steps, "
                         "timed by their own events, with the shader clock and board power sampled "
                         "in the timed half (0 = skip)")
    ap.add_argument("--tile", default=None, help="force a tile, e.g. tiled:256x256 or skinny:16x32")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (the known-size kernel that "
                         "scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                           "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of the "
                         "workload's GEMM, then of --copy-calibration 256) into "
                         "profiles/traffic_<workload>.json for --workload/--tile, and exit")
    ap.add_argument("--eager", action="store_true",
                    help="issue the K timed calls eagerly instead of replaying them from one HIP graph")
    ap.add_argument("--epilogue", default=None, metavar="PARTS",
                    help="time the fused epilogue (e.g. silu,mul or gelu,bias or scale_m,scale_n) "
                         "against the plain GEMM followed by torch elementwise ops")
    ap.add_argument("--backward-prep", action="store_true",
                    help="time transpose_2d and shuffle_b_t on the GPT-3-XL backward operands")
    ap.add_argument("--workspace-mib", type=int, default=WORKSPACE_MIB,
                    help="split-K workspace handed to the library (0: no split-K)")
    ap.add_argument("--sweep-soak", type=float, default=0.0, metavar="SECONDS",
                    help="with --sweep: time every tile in the loaded power state, its graph "
                         "replayed for SECONDS")
    ap.add_argument("--read-floor", nargs="*", default=None, metavar="WORKLOAD",
                    help="time the streaming-read probe over each workload's A and B bytes "
                         "(default: the HBM-bound workloads), one JSON line each, and exit")
    ap.add_argument("--no-hipblaslt", action="store_true",
                    help="skip the same-box hipBLASLt (torch.mm) comparison")
    ap.add_argument("--sweep", action="store_true",
                    help="time every tile of the ladder on the workload (one JSON line each) and the "
                         "selector's pick; reports the selector's regret")
    ap.add_argument("--sweep-only", default=None, metavar="REGEX",
                    help="with --sweep: time only the tiles whose name matches REGEX (a full match)")
    ap.add_argument("--regret", default=None, metavar="SWEEP_JSONL",
                    help="host only: the selector's pick against the fastest tile of every workload "
                         "in a --sweep output file")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the sharded design is described, not built).", file=sys.stderr)
        return 2
    if args.regret:               # host-only: reads sweep lines, prices with the library
        return regret_report(args.regret, args.workspace_mib)
    if args.traffic_summary:      # host-only: parses counter files
        return traffic_summary(args.workload, args.tile, *args.traffic_summary)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    name = args.workload
    M, N, K, dt = WORKLOADS[name][:4]
    if args.sweep:
        return sweep(name, args.steps, args.warmup, args.workspace_mib, args.sweep_soak, args.sweep_only)
    if args.read_floor is not None:
        return read_floor_report(args.read_floor or
                                 [n for n in WORKLOADS if bound_of(*WORKLOADS[n][:4]) == "hbm"])
    if args.backward_prep:
        return backward_prep(args.steps)
    if args.epilogue is not None:
        return epilogue_compare(name, args.epilogue, args.steps, args.workspace_mib)
    workspace = (torch.empty(args.workspace_mib << 20, dtype=torch.uint8, device="cuda")
                 if args.workspace_mib > 0 else None)
    # The decode measurement runs first: after the headline's soak the board
    # sits at its power limit with a lowered shader clock, a state a decode
    # loop (about 1 kW) does not put it in.
    secondary = None
    if not args.no_secondary and name != DECODE:
        dM, dN, dK, ddt = WORKLOADS[DECODE][:4]
        us_cold, dshuf = run_graph(DECODE, reps=60, copies=6)
        us_hot, _ = run_graph(DECODE, reps=60, copies=1)
        gb = alg_bytes(dM, dN, dK, ddt)
        secondary = {
            "workload": DECODE, "M": dM, "N": dN, "K": dK,
            "tile": dg_tile_name(dM, dN, dK, ddt),
            "us_cold": round(us_cold, 3), "GBps_cold": round(gb / (us_cold * 1e-6) / 1e9, 1),
            "frac_hbm_cold": round(gb / (us_cold * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "us_hot_mall": round(us_hot, 3), "GBps_hot_mall": round(gb / (us_hot * 1e-6) / 1e9, 1),
            "shuffle_b_us": round(dshuf, 2),
            "shuffle_b_amortized_below_1pct_after_calls": math.ceil(99.0 * dshuf / us_cold),
            # the library's streaming-read probe over the same bytes, timed
            # the same way: what any kernel reading them once would need
            "read_floor_us": _safe(lambda: round(read_floor_us((dM + dN) * dK * 2), 3)),
            "timing": "hipGraph of 60 launches, before the headline's steps; cold = 6 rotated "
                      "operand copies (541 MB)",
        }
    # No events between launches: the K calls run back to back (replayed from
    # one HIP graph unless --eager), and the event pair around them gives the
    # average launch duration (with split-K: of the GEMM and its reduction).
    r = run_timed(name, args.steps, args.warmup, tile=parse_tile(args.tile), soak=args.soak,
                  copies=args.copies or None, per_launch=False, workspace=workspace,
                  graph=not args.eager)
    ms_per_step = r["total_ms"] / args.steps
    kern_avg = r["total_ms"] * 1e3 / args.steps
    bound = bound_of(M, N, K, dt)
    if bound == "mfma":
        achieved = flops(M, N, K) / (kern_avg * 1e-6) / 1e12
        peak, unit_r = PEAK_TFLOPS[dt], "TFLOP/s"
    else:
        achieved = alg_bytes(M, N, K, dt) / (kern_avg * 1e-6) / 1e9
        peak, unit_r = PEAK_HBM_GBPS, "GB/s"
    value = flops(M, N, K) * args.steps / (r["total_ms"] * 1e-3) / 1e12
    tile = r["tile"]
    second = None
    if args.tile is None:      # the library's own plan: one launch, or two over column or row ranges
        import dense_gemm_linear_amd as dg
        _, t2, n1, m1 = dg.plan(M, N, K, dt, CUS, workspace.numel() if workspace is not None else 0)
        if t2 is not None and n1 < N:
            second = {"tile": t2.name, "first_columns": n1, "second_columns": N - n1}
        elif t2 is not None:
            second = {"tile": t2.name, "first_rows": m1, "second_rows": M - m1}
    out = {
        "metric": "GEMM TFLOP/s (2MNK/t) + % MFMA peak; HBM GB/s for M<=8 decode",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "tile": tile.name,
                   "tile_eff": round(tile.tile_eff, 4), "wq_eff": round(tile.wq_eff, 4),
                   "operand_copies_rotated": r["copies"], "pct_of_mfma_peak": None,
                   "workspace_mib": args.workspace_mib,
                   **({"second_launch": second} if second else {})},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit_r,
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "algorithmic_bytes": alg_bytes(M, N, K, dt),
                     "kernel_us_avg": round(kern_avg, 3),
                     "timing": ("HIP events around the K back-to-back calls on the kernels' stream"
                                + ("" if args.eager else ", replayed from one HIP graph")
                                + (", right after the sustained replay (board at its loaded "
                                   "power state)" if r["sustained"] else ""))},
        "shuffle_b_us": round(r["shuffle_us"], 2),
        # the preshuffle runs once per weight: the number of GEMM calls on the
        # same weight after which its cost is at most 1 % of the total
        "shuffle_b_amortized_below_1pct_after_calls":
            math.ceil(99.0 * r["shuffle_us"] / kern_avg) if kern_avg > 0 else None,
    }
    if bound == "mfma":
        out["config"]["pct_of_mfma_peak"] = round(100 * value / PEAK_TFLOPS[dt], 2)
    tr = load_traffic(name, tile.name)
    if tr:
        out["roofline"]["traffic"] = tr["hbm_bytes_per_launch"]
        out["roofline"]["traffic_detail"] = {k: tr[k] for k in ("fetch_bytes", "write_bytes",
                                                                 "fetch_factor", "write_factor",
                                                                 "source")}
    sus = r["sustained"]
    if sus:
        # the same graph replayed back to back for about --soak seconds: the
        # board at its loaded power state, timed by its own events, with the
        # shader clock sampled inside the same interval
        us = sus["per_call_us"]
        sus["value"] = round(flops(M, N, K) / (us * 1e-6) / 1e12, 2) if bound == "mfma" else \
            round(alg_bytes(M, N, K, dt) / (us * 1e-6) / 1e9, 1)
        sus["unit"] = unit_r
        sus["frac"] = round(sus["value"] / peak, 4)
        out["sustained"] = sus
        if bound == "mfma" and sus.get("gfx_mhz_mean"):
            # against the MFMA peak at the clock sampled during that interval
            out["roofline"]["frac_at_sustained_clock"] = round(
                sus["value"] / (peak * sus["gfx_mhz_mean"] / 2400.0), 4)
    if not args.no_hipblaslt and args.tile is None:
        try:
            out["hipblaslt_same_box"] = hipblaslt_same_box(name, args.steps, args.warmup, args.soak)
        except Exception as e:  # noqa: BLE001 - context only: never lose the bench line for it
            out["hipblaslt_same_box"] = {"error": f"{type(e).__name__}: {e}"[:200]}
    if secondary is not None:
        out["secondary"] = secondary
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(name)
    print(json.dumps(out), flush=True)
    return 0


def regret_report(path: str, ws_mib: int = WORKSPACE_MIB) -> int:
    """The selector's pick (at 256 CUs, with a ws_mib workspace) against the
    fastest tile of each workload in a `--sweep` output file: one JSON line per
    workload and a summary.  Host only."""
    import dense_gemm_linear_amd as dg
    res = {}
    with open(path) as f:
        for line in f:
            if line.startswith('{"sweep":'):
                d = json.loads(line)
                res.setdefault(d["sweep"], {})[d["tile"]] = d["kernel_us_median"]
    regrets = []
    for name in sorted(res):
        r = res[name]
        M, N, K, dt = WORKLOADS[name][:4]
        t = dg.select_tile(M, N, K, dt, CUS, workspace_bytes=ws_mib << 20)
        best = min(r, key=r.get)
        got = r.get(t.name)
        reg = round(got / r[best], 4) if got else None
        regrets.append(reg)
        print(json.dumps({"workload": name, "selected": t.name, "selected_us": got, "best": best,
                          "best_us": r[best], "regret": reg}))
    known = [x for x in regrets if x is not None]
    print(json.dumps({"regret_summary": path, "workloads": len(regrets),
                      "at_best": sum(1 for x in known if x == 1.0),
                      "within_5pct": sum(1 for x in known if x <= 1.05),
                      "worst": max(known) if known else None,
                      "geomean": round(math.exp(sum(math.log(x) for x in known) / len(known)), 4)
                      if known else None,
                      "unmeasured_picks": regrets.count(None)}))
    return 0


def sustained_graph_us(call, steps: int, seconds: float) -> float:
    """Per-call time of `call` in the loaded power state: `steps` calls
    captured in one HIP graph, replayed back to back for `seconds`, the
    median of the second half (sustained_with_clock)."""
    import torch
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                call(3 + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    us = sustained_with_clock(g, steps, seconds)["per_call_us"]
    del g
    return us


def sweep(name: str, steps: int, warmup: int, ws_mib: int = WORKSPACE_MIB, soak: float = 0.0,
          only: str | None = None) -> int:
    """Every feasible tile on one workload, graph-timed (`steps` launches per
    graph, median of 3 replays); prints a line per tile and a summary with
    the selector's regret (its pick's time over the best time).  soak > 0:
    each tile is timed instead in the loaded power state, its graph replayed
    for `soak` seconds (for long compute-bound workloads, whose ranking
    under the board's power limit can differ from a short burst's)."""
    import torch
    import dense_gemm_linear_amd as dg
    M, N, K, dt = WORKLOADS[name][:4]
    setup = gpu_setup(name, cold_copies(alg_bytes(M, N, K, dt)))
    tiles = dg.all_tiles(M, dt)
    # split-K variants of the rungs that leave CUs idle, one per distinct
    # slice count after the library lowers it
    ws_bytes = ws_mib << 20
    for t in list(tiles):
        if t.kernel == dg.GEMM_KERNEL_SKINNY or -(-M // t.tile_m) * -(-N // t.tile_n) >= CUS:
            continue
        seen = set()
        for S in SPLITS:
            ts = dg.with_split(t, S)
            need = dg.workspace_bytes(M, N, K, dt, ts)
            if 0 < need <= ws_bytes and need not in seen:
                seen.add(need)
                tiles.append(ts)
    # stream-K forms of the rungs that have one, for shapes filling less than
    # one round of the CUs
    for t in list(tiles):
        if t.kernel in (dg.GEMM_KERNEL_TILED, dg.GEMM_KERNEL_TILED_AB) and t.k_split <= 1 and \
                128 * 128 <= t.tile_m * t.tile_n <= 128 * 256 and \
                -(-M // t.tile_m) * -(-N // t.tile_n) < CUS:
            ts = dg.with_stream_k(t)
            need = dg.workspace_bytes(M, N, K, dt, ts)
            if 0 < need <= ws_bytes:
                tiles.append(ts)
    if only:
        import re
        tiles = [t for t in tiles if re.fullmatch(only, t.name)]
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    sets, scales, _ = setup
    res = {}
    for t in tiles:
        call = gemm_call(name, sets, scales, t, workspace)
        us = sustained_graph_us(call, steps, soak) if soak > 0 else time_graph(call, reps=steps, trials=3)
        res[t.name] = us
        print(json.dumps({"sweep": name, "tile": t.name, "kernel_us_median": round(us, 3),
                          **({"timing": f"sustained {soak} s"} if soak > 0 else {}),
                          "tflops": round(flops(M, N, K) / (us * 1e-6) / 1e12, 1),
                          "gbps": round(alg_bytes(M, N, K, dt) / (us * 1e-6) / 1e9, 1)}), flush=True)
    # the selector's single-launch pick (the sweep times single launches; a
    # two-launch plan's first tile is chosen for part of the shape only)
    pick = dg.select_tile(M, N, K, dt, CUS, workspace_bytes=ws_bytes)
    if not res:
        print(json.dumps({"sweep_summary": name, "selected": pick.name, "timed": 0}), flush=True)
        return 0
    if pick.name not in res:
        print(json.dumps({"sweep_summary": name, "selected": pick.name, "timed": len(res)}), flush=True)
        return 0
    best = min(res, key=res.get)
    print(json.dumps({"sweep_summary": name, "selected": pick.name, "selected_us": round(res[pick.name], 3),
                      "best": best, "best_us": round(res[best], 3),
                      "regret": round(res[pick.name] / res[best], 4)}), flush=True)
    return 0


def copy_calibration(mib: int) -> int:
    """Five device-to-device copies of a known size: under rocprofv3 --pmc the
    copy kernel's FETCH_SIZE and WRITE_SIZE per dispatch, against mib MiB,
    give the factor that turns those counters into HBM bytes."""
    import torch
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
    return 0


def _pmc_mean(folder: str, counter: str, kernel_substr: str) -> float:
    """Mean per-dispatch value (KiB for FETCH_SIZE / WRITE_SIZE) of `counter`
    over the dispatches of kernels whose name contains `kernel_substr`."""
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for '{kernel_substr}' under {folder}")
    return sum(vals) / len(vals)


def traffic_summary(name: str, tile_spec, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir) -> int:
    """HBM traffic of the GEMM kernel per launch: its FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by bytes / counter of a plain device copy
    of 256 MiB measured the same way."""
    import dense_gemm_linear_amd as dg
    M, N, K, dt = WORKLOADS[name][:4]
    tile = parse_tile(tile_spec) if tile_spec else dg.select_tile(M, N, K, dt, num_cus=256)
    copy_bytes = 256 * 2 ** 20
    cf = _pmc_mean(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw = _pmc_mean(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    kern = "gemm_"
    gf = _pmc_mean(fetch_dir, "FETCH_SIZE", kern)
    gw = _pmc_mean(write_dir, "WRITE_SIZE", kern)
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    t = {"workload": name, "tile": tile.name, "kernel_source_hash": kernel_source_hash(),
         "fetch_bytes": round(gf * 1024 * ff), "write_bytes": round(gw * 1024 * wf),
         "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
         "algorithmic_bytes": alg_bytes(M, N, K, dt),
         "source": "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMM kernel, "
                   "scaled by a 256 MiB device copy's bytes / counter"}
    t["hbm_bytes_per_launch"] = t["fetch_bytes"] + t["write_bytes"]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"traffic_{name}.json"), "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t), flush=True)
    return 0


def dg_tile_name(M, N, K, dt):
    import dense_gemm_linear_amd as dg
    return dg.select_tile(M, N, K, dt).name


if __name__ == "__main__":
    sys.exit(main())
