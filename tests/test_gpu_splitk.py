"""Split-K on the GPU against the oracle (C ABI, *_ws entry points).

A split-K tile runs the tiled kernels over K slices; every workgroup writes
an fp32 partial tile into the caller's workspace and a second kernel adds
the slices in increasing order, scales (e4m3) and rounds to bf16.  The
workspace is filled with 0xFF bytes (NaN as fp32) before each call, so a
partial that is read without having been written poisons the output.

Bars: bit-exact on small-integer inputs (every partial sum is an integer
below 2^24, so fp32 adds them exactly in any order); the relative Frobenius
and per-element bounds of parity.py otherwise; bitwise repeatability (the
slice order is fixed).
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
from parity import (abs_bits, check_close, check_exact, oracle_full, oracle_lines, run,
                    sample_lines)

pytestmark = pytest.mark.gpu

BF16_TILES = [dg.tiled(64, 64), dg.tiled(128, 128, 4, 32), dg.tiled(256, 128, 8),
              dg.tiled_ab(128, 128, 4, 32), dg.tiled_ab(256, 256, 8, 32), dg.tiled_pp(256, 256)]
FP8_TILES = [dg.tiled(64, 64), dg.tiled(128, 128, 4, 32), dg.tiled_ab(256, 256, 8, 32),
             dg.tiled_pp(256, 256)]
# K = 1040 bf16 is 16.25 k-tiles of 128 bytes: slices of unequal length, the
# last one holding the ragged K tail; 7 slices are lowered to 6.
BF16_SHAPE = (263, 270, 1040)
FP8_SHAPE = (200, 333, 1088)


def nan_workspace(nbytes: int) -> torch.Tensor:
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


def split_run(dt, A, B, tile, **kw):
    M, K = A.shape
    N = B.shape[0]
    nbytes = dg.workspace_bytes(M, N, K, dt, tile)
    assert nbytes > 0, f"{tile.name} does not split {M}x{N}x{K}"
    print(f"[split {dt} {tile.name} {M}x{N}x{K} ws={nbytes}]", flush=True)
    C, ok = run(dt, A, B, tile=tile, workspace=nan_workspace(nbytes), **kw)
    assert ok, "guard band written"
    return C


@pytest.mark.parametrize("S", [2, 3, 7])
@pytest.mark.parametrize("tile", BF16_TILES, ids=lambda t: t.name)
def test_split_bf16(tile, S):
    M, N, K = BF16_SHAPE
    t = dg.with_split(tile, S)
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=70 + S)
    check_exact(split_run("bf16", A, B, t), oracle_full("bf16", A, B), t.name)
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=80 + S)
    check_close("bf16", split_run("bf16", A, B, t), oracle_full("bf16", A, B),
                oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)), K, what=t.name)


@pytest.mark.parametrize("S", [2, 5])
@pytest.mark.parametrize("tile", FP8_TILES, ids=lambda t: t.name)
def test_split_fp8(tile, S):
    M, N, K = FP8_SHAPE
    t = dg.with_split(tile, S)
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=90 + S, smallint=True)
    for s1, s2 in ((1.0, 1.0), (2.0 ** -3, 2.0 ** 2)):
        C = split_run("fp8", A, B, t, sa=s1, sb=s2)
        check_exact(C, oracle_full("fp8", A, B, s1, s2), f"{t.name} scales {s1} {s2}")
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=95 + S)
    C = split_run("fp8", A, B, t, sa=sa, sb=sb)
    check_close("fp8", C, oracle_full("fp8", A, B, sa, sb),
                oracle_full("fp8", abs_bits("fp8", A), abs_bits("fp8", B)), K, scale=sa * sb,
                what=t.name)


@pytest.mark.parametrize("tile", [dg.tiled(128, 128, 4, 32), dg.tiled_pp(256, 256)],
                         ids=lambda t: t.name)
def test_split_short_k(tile):
    """More slices asked for than k-tiles: one k-tile per slice."""
    M, N, K = 90, 200, 128
    t = dg.with_split(tile, 8)
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=11)
    check_exact(split_run("bf16", A, B, t), oracle_full("bf16", A, B), t.name)


def test_split_repeatable_and_odd_ldc():
    M, N, K = BF16_SHAPE
    t = dg.with_split(dg.tiled_ab(128, 128, 4, 32), 4)
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=12)
    C1 = split_run("bf16", A, B, t)
    C2 = split_run("bf16", A, B, t, ldc=N + 7, col0=3)
    assert np.array_equal(C1, C2), "split-K results differ between runs"


TP_SHAPES = [("bf16", 597, 1376, 4096, 61), ("bf16", 597, 4096, 1376, 63),
             ("fp8", 597, 1376, 4096, 64)]


@pytest.mark.parametrize("dt,M,N,K,cfg", TP_SHAPES, ids=lambda v: str(v))
def test_selected_with_workspace_sampled(dt, M, N, K, cfg):
    """Full-size tensor-parallel shard shapes, tile chosen by the library with
    a 64 MiB workspace; whole rows and columns checked against the oracle."""
    ws = nan_workspace(64 << 20)
    t = dg.select_tile(M, N, K, dt, workspace_bytes=ws.numel())
    print(f"[selected {dt} {M}x{N}x{K}: {t.name}]", flush=True)
    if dt == "bf16":
        A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", cfg, 1.0, 0.02)
        sa = sb = 1.0
    else:
        A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=cfg)
    C, ok = run(dt, A, B, sa=sa, sb=sb, workspace=ws)
    assert ok
    rows, cols = sample_lines(M), sample_lines(N)
    ms, ns, vals, absv = oracle_lines(dt, A, B, rows, cols, sa * sb)
    check_close(dt, C[ms, ns][None, :], vals[None, :], absv[None, :], K, scale=sa * sb,
                what=f"{dt} {M}x{N}x{K} {t.name}")


def test_two_launches_with_split_remainder():
    """4096 x 12480 x 2048 with the bench's 64 MiB workspace: the chosen
    256 x 256 tile would run 3 full rounds and 32 tiles more, so the first
    12288 columns run with it and the other 192 as a split-K GEMM that uses
    the workspace (gemm_plan).  Whole rows and whole columns on both sides of
    the launch boundary and of tile boundaries, bit-exact on small integers."""
    M, N, K = 4096, 12480, 2048
    ws = nan_workspace(64 << 20)
    first, second, n1, _ = dg.plan(M, N, K, "bf16", 256, ws.numel())
    print(f"[two launches {M}x{N}x{K}: {first.name} x {n1} + {second and second.name}]", flush=True)
    assert second is not None and second.k_split > 1 and n1 == 12288, "shape no longer splits"
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=213)
    C, ok = run("bf16", A, B, workspace=ws)
    assert ok
    rows = sample_lines(M)
    cols = np.unique(np.concatenate([sample_lines(N), np.arange(n1 - 3, n1 + 3), np.arange(N - 3, N)]))
    ms, ns, vals, _ = oracle_lines("bf16", A, B, rows, cols)
    check_exact(C[ms, ns][None, :], vals[None, :], "two launches, split-K remainder")


@pytest.mark.parametrize("ws_mib", [0, 128])
def test_two_launches_over_rows(ws_mib):
    """8704 x 2048 x 1024: 272 tiles of 256 x 256, one round and 16 tiles
    more; the rows [0, 8192) run with that tile and the other 512 rows as a
    second GEMM (gemm_plan's row split).  Whole rows on both sides of the
    launch boundary, whole columns, bit-exact on small integers."""
    M, N, K = 8704, 2048, 1024
    ws = nan_workspace(ws_mib << 20) if ws_mib else None
    first, second, n1, m1 = dg.plan(M, N, K, "bf16", 256, ws.numel() if ws is not None else 0)
    print(f"[row split {M}x{N}x{K} ws {ws_mib} MiB: {first.name} x {m1} rows + "
          f"{second and second.name}]", flush=True)
    assert second is not None and m1 == 8192 and n1 == N, "shape no longer splits by rows"
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=214)
    C, ok = run("bf16", A, B, workspace=ws)
    assert ok
    rows = np.unique(np.concatenate([sample_lines(M), np.arange(m1 - 3, m1 + 3), np.arange(M - 3, M)]))
    cols = sample_lines(N)
    ms, ns, vals, _ = oracle_lines("bf16", A, B, rows, cols)
    check_exact(C[ms, ns][None, :], vals[None, :], "two launches over rows")


def test_two_launches_over_rows_split_remainder():
    """10240 x 2048 x 8192 (the GPT-3-XL input gradient) with a 128 MiB
    workspace: 8192 rows on the 256 x 256 tile, the other 2048 as a split-K
    GEMM that uses the workspace.  Sampled rows and columns on both sides of
    the boundary against the oracle: bit-exact on small integers."""
    M, N, K = 10240, 2048, 8192
    ws = nan_workspace(128 << 20)
    first, second, n1, m1 = dg.plan(M, N, K, "bf16", 256, ws.numel())
    print(f"[row split {M}x{N}x{K}: {first.name} x {m1} rows + {second and second.name}]", flush=True)
    assert second is not None and second.k_split > 1 and m1 == 8192, "shape no longer splits by rows"
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=215)
    C, ok = run("bf16", A, B, workspace=ws)
    assert ok
    rows = np.unique(np.concatenate([sample_lines(M, n_random=3), np.arange(m1 - 2, m1 + 2)]))
    cols = sample_lines(N, n_random=3)
    ms, ns, vals, _ = oracle_lines("bf16", A, B, rows, cols)
    check_exact(C[ms, ns][None, :], vals[None, :], "two launches over rows, split-K remainder")
