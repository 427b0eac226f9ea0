"""e4m3 GEMM with per-tensor scales on the GPU against the oracle (C ABI).

Inputs: N(0, 1) quantised per tensor to amax 448 (the fp8 workloads), and a
small-integer variant whose values are exact e4m3 codes: with scales 1 and
with the power-of-two scales 2^-3, 2^2 the output is bit-exact.  The general
bound is 3e-2 relative Frobenius against the oracle on the same e4m3 bytes
with the scales applied, plus the per-element bound of parity.py.
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
from parity import abs_bits, check_close, check_close_full, check_exact, oracle_full, run

pytestmark = pytest.mark.gpu

WORKLOADS = {"cfg5_4096cube": (4096, 4096, 4096, 5), "cfg5_32x4096": (32, 4096, 4096, 51)}
SMALL_SHAPES = [(128, 256, 128), (33, 65, 64), (1, 16, 64), (263, 270, 192), (597, 600, 256)]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_full(shape):
    M, N, K = shape
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=M + 3 * N)
    C, ok = run("fp8", A, B, sa=sa, sb=sb)
    assert ok
    check_close("fp8", C, oracle_full("fp8", A, B, sa, sb),
                oracle_full("fp8", abs_bits("fp8", A), abs_bits("fp8", B)), K, scale=sa * sb,
                what=str(shape))
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=M + 3 * N, smallint=True)
    for (s1, s2) in ((1.0, 1.0), (2.0 ** -3, 2.0 ** 2)):
        C, ok = run("fp8", A, B, sa=s1, sb=s2)
        assert ok
        check_exact(C, oracle_full("fp8", A, B, s1, s2), f"{shape} smallint scales {s1},{s2}")


BENCH_WORKSPACE = 128 << 20   # the split-K / stream-K workspace bench.py hands the library


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("smallint", [False, True], ids=["general", "smallint"])
def test_workload_shapes_every_element(name, smallint):
    """Every output element against the oracle's whole product, on the
    library's plan without a workspace and, where it differs, on the plan
    bench.py times with its 128 MiB workspace."""
    M, N, K, cfg = WORKLOADS[name]
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=cfg, smallint=smallint)
    if smallint:
        sa, sb = 2.0 ** -3, 2.0 ** 2
    print(f"[gemm_fp8 {name} {M}x{N}x{K} smallint={smallint}: oracle product]", flush=True)
    ref = oracle_full("fp8", A, B, sa, sb)
    runs = [(0, dg.plan(M, N, K, "fp8", 256, 0)[0])]
    t_ws = dg.plan(M, N, K, "fp8", 256, BENCH_WORKSPACE)[0]
    if t_ws.name != runs[0][1].name:
        runs.append((BENCH_WORKSPACE, t_ws))
    for ws, tile in runs:
        print(f"[gemm_fp8 {name} ws={ws >> 20} MiB tile={tile.name}]", flush=True)
        workspace = torch.full((ws,), 0xFF, dtype=torch.uint8, device="cuda") if ws else None
        C, ok = run("fp8", A, B, sa=sa, sb=sb, workspace=workspace)
        assert ok, "guard band written"
        if smallint:
            check_exact(C, ref, f"{name} {tile.name}")
        else:
            check_close_full("fp8", C, ref, A, B, K, scale=sa * sb, what=f"{name} {tile.name}")


@pytest.mark.parametrize("tile", dg.ladder_tiles("fp8"), ids=lambda t: t.name)
def test_every_ladder_tile(tile):
    M, N, K = 263, 270, 192
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=19, smallint=True)
    C, ok = run("fp8", A, B, tile=tile, sa=0.5, sb=4.0)
    assert ok
    check_exact(C, oracle_full("fp8", A, B, 0.5, 4.0), tile.name)


@pytest.mark.parametrize("tile", dg.ladder_tiles("fp8"), ids=lambda t: t.name)
def test_every_ladder_tile_short_k(tile):
    """1 to 6 k-tiles (fewer than the pipeline stages for some rungs), three
    runs each: a missing wait shows up as stale LDS data in some runs only."""
    M, N = 128, 256
    for K in (64, 128, 192, 256, 384):
        A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=K + 7, smallint=True)
        ref = oracle_full("fp8", A, B)
        for rep in range(3):
            C, ok = run("fp8", A, B, tile=tile)
            assert ok
            check_exact(C, ref, f"{tile.name} K={K} run {rep}")


# The 4-wave 256 x 256 rung with 32 x 32 atoms and four 64-byte stages runs on
# the kernel that loads A in k-tile pairs of whole 128-byte lines into three
# pair stages: K counts whose last pair is half full or empty, a main loop
# followed by 1-3 tail phases, partial row and column tiles, and repeated
# runs (a stage reused too early shows up as stale data in some runs only).
@pytest.mark.parametrize("M,N,K", [(300, 520, 448), (513, 264, 576), (256, 256, 1088),
                                   (40, 300, 832), (257, 512, 64), (100, 300, 192),
                                   (600, 700, 4160)],
                         ids=lambda v: str(v))
def test_whole_line_a_rung(M, N, K):
    tile = dg.tiled_ab(256, 256, 4, 32, stages=4, tile_k=64)
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=M + N + K, smallint=True)
    ref = oracle_full("fp8", A, B, 0.5, 2.0)
    for rep in range(3):
        C, ok = run("fp8", A, B, tile=tile, sa=0.5, sb=2.0)
        assert ok, "guard band written"
        check_exact(C, ref, f"{tile.name} {M}x{N}x{K} run {rep}")


@pytest.mark.parametrize("tm,tn,w", dg.SKINNY_LADDER)
def test_every_skinny_tile(tm, tn, w):
    M, N, K = tm - 3, 270, 320
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=20 + tm, smallint=True)
    C, ok = run("fp8", A, B, tile=dg.skinny(tm, tn, w))
    assert ok
    check_exact(C, oracle_full("fp8", A, B), f"skinny{tm}x{tn}w{w}")


@pytest.mark.parametrize("K", [64, 192, 320])
def test_k_tails(K):
    M, N = 40, 90
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=K, smallint=True)
    for tile in (None, dg.tiled(64, 64), dg.tiled(128, 256), dg.tiled(256, 128, 8),
                 dg.tiled_ab(256, 128, 4), dg.skinny(48, 32), dg.tiled(128, 128, 4, 32),
                 dg.tiled_ab(256, 256, 8, 32), dg.tiled_ab(128, 256, 4, 32), dg.tiled_pp(256, 256)):
        C, ok = run("fp8", A, B, tile=tile)
        assert ok
        check_exact(C, oracle_full("fp8", A, B), f"K={K} {tile}")


def test_guard_band_odd_ldc():
    M, N, K = 75, 333, 128
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=3, smallint=True)
    for ldc, col0 in ((N, 0), (N + 9, 2), (N + 16, 8)):
        C, ok = run("fp8", A, B, ldc=ldc, col0=col0)
        assert ok
        check_exact(C, oracle_full("fp8", A, B), f"ldc={ldc} col0={col0}")


@pytest.mark.parametrize("tile", [dg.tiled(128, 128, 4, 32), dg.tiled_ab(256, 256, 8, 32),
                                  dg.tiled_pp(256, 256)], ids=lambda t: t.name)
def test_odd_pitch_large_tiles(tile):
    """Rows at odd 2-byte phases on the large e4m3 rungs, several tiles and a
    ragged edge in both directions."""
    M, N, K = 530, 2 * 256 + 45, 192
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=5, smallint=True)
    for ldc, col0 in ((N + 1, 0), (N + 10, 5)):
        C, ok = run("fp8", A, B, tile=tile, sa=0.5, sb=2.0, ldc=ldc, col0=col0)
        assert ok
        check_exact(C, oracle_full("fp8", A, B, 0.5, 2.0), f"{tile.name} ldc={ldc} col0={col0}")
