"""Fit select_tile's per-rung cost constants from measured tile sweeps.

Input: JSON lines written by ``bench.py --sweep`` (one per workload and rung:
{"sweep": workload, "tile": rung name, "kernel_us_median": t}), by default
``calibration/mi355x_sweep.jsonl``.  For each element type and tiled / A+B
rung, the kernel time is modelled as

    t = a * n_cu * K_bytes / 1000 + b * n_cu + c     (microseconds)

with n_cu = ceil(tiles / CUs) the tiles the busiest CU runs (wave
quantization, TraceLens GEMM analysis page, "Wave quantization efficiency"),
K_bytes = K * element bytes (the K loop), and b, c the per-tile and per-launch
fixed costs (prologue, epilogue, launch).  a, b, c >= 0 are fitted by
non-negative least squares over the workloads the rung was measured on.
Writes ``csrc/calibration.inc`` (a C table select_tile includes).

    python dense_gemm_linear_amd/calibrate.py [sweep.jsonl ...]
"""
from __future__ import annotations

import json
import math
import os
import re
import sys

import numpy as np
from scipy.optimize import nnls

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CUS = 256


def workloads():
    sys.path.insert(0, ROOT)
    import bench
    return bench.WORKLOADS


SKINNY = re.compile(r"skinny(\d+)x(\d+)(?:w(\d+))?$")
NAME = re.compile(r"(tiled|ab|pp)(\d+)x(\d+)(?:w(\d+))?(?:a(\d+))?s(\d+)k(\d+)(?:sk(\d+))?$")


def parse(name: str):
    """Rung fields from a tile name, or None for skinny rungs."""
    m = NAME.match(name)
    if not m:
        return None
    kind, tm, tn, w, a, st, tk, sk = m.groups()
    return {"kernel": {"tiled": 0, "ab": 2, "pp": 3}[kind], "tm": int(tm), "tn": int(tn),
            "waves": int(w or (8 if kind == "pp" else 4)), "atom": int(a or 16), "stages": int(st),
            "tile_k": int(tk), "k_split": int(sk or 1)}


def split_plan(M, N, K, e, ktb, k_split):
    """(slices, k-tiles per slice, ldw) as the library lowers k_split."""
    nkt = math.ceil(K * e / ktb)
    want = max(1, min(k_split, nkt))
    per = math.ceil(nkt / want)
    return math.ceil(nkt / per), per, math.ceil(N / 4) * 4


# select_tile drops a tile whose padded output exceeds this multiple of the
# real one (unless nothing else fits); the fit uses the same rule, so a rung's
# cost model is fitted on the shapes where it competes
PAD_LIMIT = 1.25


def load_points(paths):
    """(rung key, features, split features, t) per tiled sweep line and
    (skinny key, features, t) per skinny line."""
    wl = workloads()
    pts, sk = [], []
    for p in paths:
        for line in open(p):
            d = json.loads(line)
            M, N, K, dt = wl[d["sweep"]][:4]
            e = 2 if dt == "bf16" else 1
            t = d["kernel_us_median"]
            m = SKINNY.match(d["tile"])
            if m:
                tm, tn, w = int(m.group(1)), int(m.group(2)), int(m.group(3) or 4)
                nwg = math.ceil(math.ceil(N / 16) / (tn // 16))
                per_cu = math.ceil(nwg / CUS)
                wg_mb = (tn * K * e + tm * K * e) / 1e6
                total_mb = (math.ceil(N / 16) * 16 * K * e + M * K * e + 2 * M * N) / 1e6
                sk.append(((dt, tm, tn, w), [per_cu * wg_mb, total_mb, 1.0], t))
                continue
            r = parse(d["tile"])
            if r is None:
                continue
            ktb = r["tile_k"] * e
            key = (dt, r["kernel"], r["tm"], r["tn"], r["waves"], r["atom"], r["stages"], ktb)
            tiles = math.ceil(M / r["tm"]) * math.ceil(N / r["tn"])
            if tiles * r["tm"] * r["tn"] > PAD_LIMIT * M * N:
                continue   # screened out by select_tile's padding rule: not a candidate here
            S, per, ldw = split_plan(M, N, K, e, ktb, r["k_split"])
            kbytes = K * e if S == 1 else per * ktb
            ncu = math.ceil(tiles * S / CUS)
            extra = [0.0, 0.0, 0.0] if S == 1 else \
                [ncu * r["tm"] * r["tn"] * 4 / 1e6, (S * M * ldw * 4 + 2 * M * N) / 1e6, 1.0]
            total_mb = (M * K * e + N * K * e + 2 * M * N) / 1e6
            pts.append((key, [ncu * kbytes / 1000.0, ncu, total_mb, 1.0], extra, t))
    return pts, sk


def fit(paths):
    """Three fits, all non-negative least squares:
    - per rung a, b, g, c of t = a * n_cu * K_bytes / 1000 + b * n_cu
      + g * MB + c (MB: A, B and C bytes / 1e6) from its one-pass points (the
      model one-pass candidates are priced with);
    - a second set per rung fitted jointly over one-pass and split points,
      with three split-K costs shared by all rungs that only split runs pay:
          d * n_cu * tile_m * tile_n * 4 / 1e6    (fp32 partial stores per CU)
        + r1 * (S * M * ldw * 4 + 2 * M * N) / 1e6  (the reduction's traffic)
        + r0                                      (its launch),
      weighted by 1 / t (relative error ranks candidates); split candidates
      are priced with it, since it is pinned at the short K of one slice;
    - per skinny rung t = a * per_cu * MB_per_workgroup + b * MB_total + c."""
    pts, sk = load_points(paths)
    keys = sorted({k for k, _, x, _ in pts if x[2] == 0.0})
    plain = {}
    for k in keys:
        f = [(ff, t) for kk, ff, x, t in pts if kk == k and x[2] == 0.0]
        plain[k] = (nnls(np.array([a for a, _ in f]), np.array([t for _, t in f]))[0], len(f))
    F = 4
    col = {k: F * i for i, k in enumerate(keys)}
    rows = [(k, f, x, t) for k, f, x, t in pts if k in col]
    X = np.zeros((len(rows), F * len(keys) + 3))
    y = np.zeros(len(rows))
    for i, (k, f, x, t) in enumerate(rows):
        X[i, col[k]:col[k] + F] = f
        X[i, -3:] = x
        y[i] = t
    w = 1.0 / np.maximum(y, 1.0)
    coef, _ = nnls(X * w[:, None], y * w)
    rungs = [(k, plain[k][0], coef[col[k]:col[k] + F], plain[k][1]) for k in keys]
    n_split = sum(1 for r in rows if r[2][2] == 1.0)
    skinny = []
    for k in sorted({k for k, _, _ in sk}):
        f = [(ff, t) for kk, ff, t in sk if kk == k]
        skinny.append((k, nnls(np.array([a for a, _ in f]), np.array([t for _, t in f]))[0], len(f)))
    return rungs, (coef[-3:], n_split), skinny


def measured_best(paths):
    """Per swept shape, the fastest measured tile: (dt, M, N, K, tile fields)."""
    wl = workloads()
    best = {}
    for p in paths:
        for line in open(p):
            d = json.loads(line)
            key = d["sweep"]
            if key not in best or d["kernel_us_median"] < best[key][1]:
                best[key] = (d["tile"], d["kernel_us_median"])
    out = []
    for name, (tile, us) in sorted(best.items()):
        M, N, K, dt = wl[name][:4]
        m = SKINNY.match(tile)
        if m:
            w = int(m.group(3) or 4)
            f = (1, int(m.group(1)), int(m.group(2)), 0, 16, w, w, 0)
        else:
            r = parse(tile)
            f = (r["kernel"], r["tm"], r["tn"], r["tile_k"], r["atom"], r["waves"], r["k_split"],
                 r["stages"])
        out.append((0 if dt == "bf16" else 1, M, N, K, f, us, tile))
    return out


def emit(fits, path, table=()):
    rungs, ((d_st, r1, r0), n_split), skinny = fits
    lines = ["// Generated by calibrate.py from measured MI355X tile sweeps; do not edit.",
             "// {dtype, kernel, tile_m, tile_n, waves, atom, stages, k-tile bytes, a, b, g, c,",
             "//  a, b, g, c of the split-K set, one-pass points}:",
             "// t_us = a * n_cu * K_bytes / 1000 + b * n_cu + g * (A + B + C bytes) / 1e6 + c",
             "static const RungCalib kRungCalib[] = {"]
    for (dt, kern, tm, tn, w, atom, st, ktb), (a, b, g, c), (a2, b2, g2, c2), n in rungs:
        d = 0 if dt == "bf16" else 1
        lines.append(f"    {{{d}, {kern}, {tm}, {tn}, {w}, {atom}, {st}, {ktb}, "
                     f"{a:.5f}f, {b:.5f}f, {g:.5f}f, {c:.5f}f, "
                     f"{a2:.5f}f, {b2:.5f}f, {g2:.5f}f, {c2:.5f}f, {n}}},")
    lines.append("};")
    lines += ["// split-K beyond the rung's own model: d * n_cu * partial-tile MB + r1 * reduce MB + r0",
              "// {d, r1, r0, points}",
              f"static const SplitCalib kSplitCalib = {{{d_st:.5f}f, {r1:.5f}f, {r0:.5f}f, {n_split}}};",
              "// skinny rungs {dtype, tile_m, tile_n, waves, a, b, c, points}:",
              "// t_us = a * per_cu * MB_per_workgroup + b * MB_total + c",
              "static const SkinnyCalib kSkinnyCalib[] = {"]
    for (dt, tm, tn, w), (a, b, c), n in skinny:
        d = 0 if dt == "bf16" else 1
        lines.append(f"    {{{d}, {tm}, {tn}, {w}, {a:.5f}f, {b:.5f}f, {c:.5f}f, {n}}},")
    lines.append("};")
    lines += ["// measured best tile per swept shape, used for exact matches:",
              "// {dtype, M, N, K, kernel, tile_m, tile_n, tile_k, atom, waves, k_split, lds_stages,",
              "//  measured us}",
              "static const MeasuredBest kMeasuredBest[] = {"]
    for d, M, N, K, (kern, tm, tn, tk, atom, w, ks, st), us, name in table:
        lines.append(f"    {{{d}, {M}, {N}, {K}, {kern}, {tm}, {tn}, {tk}, {atom}, {w}, {ks}, {st}, "
                     f"{us:.3f}f}},   // {name}")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    paths = sys.argv[1:] or [os.path.join(HERE, "calibration", "mi355x_sweep.jsonl")]
    fits = fit(paths)
    emit(fits, os.path.join(HERE, "csrc", "calibration.inc"), measured_best(paths))
    (d_st, r1, r0), n = fits[1]
    print(f"{len(fits[0])} rungs, {len(fits[2])} skinny rungs calibrated; split-K from {n} points: "
          f"{d_st:.3f} us per MB of partials per CU, {r1:.3f} us per MB reduced, {r0:.2f} us launch")
