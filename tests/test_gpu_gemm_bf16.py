"""bf16 GEMM on the GPU against the oracle, through the C ABI.

Small shapes and full workload shapes: every output compared with the
oracle's product.  Small-integer inputs are bit-exact; general inputs
meet the relative Frobenius bound 2e-3 and the per-element bound of parity.py.
"""
import functools

import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
import oracle
from parity import check_close, check_close_full, check_exact, oracle_full, run, abs_bits

pytestmark = pytest.mark.gpu

# (M, N, K, distribution of A, sigma A, distribution of B, sigma B, config id)
WORKLOADS = {
    "cfg2_4096cube": (4096, 4096, 4096, "normal", 0.02, "normal", 0.02, 2),
    "cfg3_prefill": (597, 11008, 4096, "normal", 1.0, "normal", 0.02, 3),
    "cfg3_decode": (1, 11008, 4096, "normal", 1.0, "normal", 0.02, 3),
    "cfg4_1x11008": (1, 11008, 4096, "normal", 1.0, "normal", 1.0, 41),
    "cfg4_8x4096": (8, 4096, 4096, "normal", 1.0, "normal", 1.0, 42),
    "cfg4_48x4096": (48, 4096, 4096, "normal", 1.0, "normal", 1.0, 43),
    "cfg4_3402": (3402, 4096, 1024, "normal", 1.0, "normal", 1.0, 44),
    "cfg4_lmhead": (1024, 50257, 512, "normal", 1.0, "normal", 1.0, 45),
    "cfg4_2048x11007": (2048, 11007, 1024, "normal", 1.0, "normal", 1.0, 46),
    "cfg4_4095": (4095, 4095, 1024, "normal", 1.0, "normal", 1.0, 47),
    "cfg4_528": (528, 528, 1024, "normal", 1.0, "normal", 1.0, 48),
}

SMALL_SHAPES = [(128, 256, 128), (127, 512, 512), (512, 64, 512), (33, 65, 48), (1, 16, 16),
                (17, 33, 80), (597, 600, 256), (263, 270, 176), (48, 300, 144), (64, 64, 64)]


@functools.lru_cache(maxsize=4)
def inputs(M, N, K, da, sa, db, sb, cfg, smallint=False):
    if smallint:
        return datagen.make_bf16_pair(M, N, K, "smallint", "smallint", cfg + 500)
    return datagen.make_bf16_pair(M, N, K, da, db, cfg, sa, sb)


def test_config1_uniform_and_smallint():
    M, N, K = 128, 256, 128
    A, B = datagen.make_bf16_pair(M, N, K, "uniform", "uniform", config=1)
    C, ok = run("bf16", A, B)
    assert ok
    check_close("bf16", C, oracle_full("bf16", A, B),
                oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)), K, what="cfg1")
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=1)
    C, ok = run("bf16", A, B)
    assert ok
    check_exact(C, oracle_full("bf16", A, B), "cfg1 smallint")


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_full(shape):
    M, N, K = shape
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=M * 7 + N)
    C, ok = run("bf16", A, B)
    assert ok
    check_close("bf16", C, oracle_full("bf16", A, B),
                oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)), K, what=str(shape))
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=M * 7 + N)
    C, ok = run("bf16", A, B)
    assert ok
    check_exact(C, oracle_full("bf16", A, B), f"{shape} smallint")


BENCH_WORKSPACE = 128 << 20   # the split-K / stream-K workspace bench.py hands the library


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("smallint", [False, True], ids=["general", "smallint"])
def test_workload_shapes_every_element(name, smallint):
    """Every output element of the full workload against the oracle's whole
    product (computed once per case on the host's threads): on the library's
    plan without a workspace, and, where it differs, on the plan bench.py
    times with its 128 MiB workspace (split-K or stream-K; the workspace
    NaN-poisoned first)."""
    M, N, K, da, sa, db, sb, cfg = WORKLOADS[name]
    A, B = inputs(M, N, K, da, sa, db, sb, cfg, smallint)
    print(f"[gemm_bf16 {name} {M}x{N}x{K} smallint={smallint}: oracle product]", flush=True)
    ref = oracle_full("bf16", A, B)
    runs = [(0, dg.plan(M, N, K, "bf16", 256, 0)[0])]
    t_ws = dg.plan(M, N, K, "bf16", 256, BENCH_WORKSPACE)[0]
    if t_ws.name != runs[0][1].name:
        runs.append((BENCH_WORKSPACE, t_ws))
    for ws, tile in runs:
        print(f"[gemm_bf16 {name} ws={ws >> 20} MiB tile={tile.name}]", flush=True)
        workspace = torch.full((ws,), 0xFF, dtype=torch.uint8, device="cuda") if ws else None
        C, ok = run("bf16", A, B, workspace=workspace)
        assert ok, "guard band written"
        if smallint:
            check_exact(C, ref, f"{name} {tile.name}")
        else:
            check_close_full("bf16", C, ref, A, B, K, what=f"{name} {tile.name}")


EVERY_SHAPE = (263, 270, 176)   # divides no tile in M, N or the 64-element k-tile


@pytest.mark.parametrize("tile", dg.ladder_tiles("bf16"), ids=lambda t: t.name)
def test_every_ladder_tile(tile):
    M, N, K = EVERY_SHAPE
    for smallint in (False, True):
        A, B = datagen.make_bf16_pair(M, N, K, "smallint" if smallint else "normal",
                                      "smallint" if smallint else "normal", config=9)
        C, ok = run("bf16", A, B, tile=tile)
        assert ok, "guard band written"
        Cref = oracle_full("bf16", A, B)
        if smallint:
            check_exact(C, Cref, tile.name)
        else:
            check_close("bf16", C, Cref, oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)),
                        K, what=tile.name)


@pytest.mark.parametrize("tile", dg.ladder_tiles("bf16"), ids=lambda t: t.name)
def test_every_ladder_tile_short_k(tile):
    """1 to 5 k-tiles: K loops that end inside the prologue or run only the
    tail phases (fewer k-tiles than pipeline stages).  Each case runs three
    times: a missing wait shows up as stale LDS data in some runs only."""
    M, N = 128, 256
    for K in (64, 128, 192, 256, 320):
        A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=K + 3)
        ref = oracle_full("bf16", A, B)
        for rep in range(3):
            C, ok = run("bf16", A, B, tile=tile)
            assert ok, "guard band written"
            check_exact(C, ref, f"{tile.name} K={K} run {rep}")


@pytest.mark.parametrize("tm,tn,w", dg.SKINNY_LADDER)
@pytest.mark.parametrize("M", [1, 13, 16, 17, 31, 47, 48, 64])
def test_every_skinny_tile(tm, tn, w, M):
    if M > tm:
        pytest.skip("tile rows do not cover M")
    N, K = 270, 176
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=10 + M)
    C, ok = run("bf16", A, B, tile=dg.skinny(tm, tn, w))
    assert ok
    check_exact(C, oracle_full("bf16", A, B), f"skinny{tm}x{tn}w{w} M={M}")


@pytest.mark.parametrize("K", [16, 48, 80, 144, 64, 128])
@pytest.mark.parametrize("tile", [None, dg.tiled(64, 64), dg.tiled(256, 128), dg.tiled(256, 128, 8),
                                  dg.tiled_ab(256, 128, 4), dg.tiled_ab(128, 128, 4), dg.skinny(32, 16),
                                  dg.tiled(128, 128, 4, 32), dg.tiled(256, 256, 8, 32),
                                  dg.tiled_ab(256, 256, 8, 32), dg.tiled_ab(128, 128, 4, 32),
                                  dg.tiled_pp(256, 256)],
                         ids=["auto", "t64x64", "t256x128", "t256x128w8", "ab256x128", "ab128x128",
                              "s32x16", "t128x128a32", "t256x256w8a32", "ab256x256w8a32",
                              "ab128x128a32", "pp256x256"])
def test_k_tails(K, tile):
    M, N = 30, 100
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=K)
    C, ok = run("bf16", A, B, tile=tile)
    assert ok
    check_exact(C, oracle_full("bf16", A, B), f"K={K}")


@pytest.mark.parametrize("M,N", [(75, 11007 % 1000), (13, 333), (300, 270)])
@pytest.mark.parametrize("ldc_extra,col0", [(0, 0), (13, 0), (7, 3), (8, 8)])
def test_guard_band_and_ldc(M, N, ldc_extra, col0):
    K = 96
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=M + N)
    C, ok = run("bf16", A, B, ldc=N + col0 + ldc_extra, col0=col0)
    assert ok, "wrote outside the M x N view"
    check_exact(C, oracle_full("bf16", A, B), f"ldc+{ldc_extra} col0={col0}")


ODD_PITCH_TILES = [dg.tiled(64, 64), dg.tiled(256, 128, 8), dg.tiled(128, 128, 4, 32),
                   dg.tiled(128, 256, 4, 32), dg.tiled(256, 256, 8, 32), dg.tiled_ab(256, 128, 4),
                   dg.tiled_ab(256, 128, 8, 32), dg.tiled_ab(128, 128, 4, 32),
                   dg.tiled_ab(256, 256, 8, 32), dg.tiled_pp(256, 256)]


@pytest.mark.parametrize("ldc_extra,col0", [(1, 0), (4, 3), (0, 7), (6, 2)])
@pytest.mark.parametrize("tile", ODD_PITCH_TILES, ids=lambda t: t.name)
def test_odd_pitch_every_family(tile, ldc_extra, col0):
    """C rows at every 2-byte phase: each row segment is staged at its own
    phase, whole 16-byte pieces go out aligned and the two shared end pieces
    element by element.  Three column tiles and a ragged one, three row tiles."""
    M, N, K = 530, 2 * 256 + 45, 96
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=ldc_extra + 10 * col0)
    C, ok = run("bf16", A, B, tile=tile, ldc=N + col0 + ldc_extra, col0=col0)
    assert ok, "wrote outside the M x N view"
    check_exact(C, oracle_full("bf16", A, B), f"{tile.name} ldc+{ldc_extra} col0={col0}")


@functools.lru_cache(maxsize=1)
def lmhead_smallint():
    """Small-integer lm_head inputs and their oracle product (shared by cases)."""
    A, B = datagen.make_bf16_pair(1024, 50257, 512, "smallint", "smallint", config=211)
    return A, B, oracle_full("bf16", A, B)


@pytest.mark.parametrize("ldc_extra,col0", [(0, 0), (3, 1)])
def test_ragged_last_round_two_launches(ldc_extra, col0):
    """1024 x 50257 x 512 (lm_head): the chosen 256 x 256 tile would run 3
    full rounds of 256 tiles and a fourth of 20, so the library runs the first
    49152 columns with it and the other 1105 as a second GEMM with a tile of
    their own (gemm_plan).  Every output against the oracle, bit-exact."""
    M, N, K = 1024, 50257, 512
    first, second, n1, _ = dg.plan(M, N, K, "bf16", 256, 0)
    print(f"[two launches {M}x{N}x{K}: {first.name} x {n1} + {second and second.name}]", flush=True)
    assert second is not None and n1 == 49152, "shape no longer splits"
    A, B, ref = lmhead_smallint()
    C, ok = run("bf16", A, B, ldc=N + col0 + ldc_extra, col0=col0)
    assert ok, "wrote outside the M x N view"
    check_exact(C, ref, f"two launches ldc+{ldc_extra} col0={col0}")


def test_repeatable():
    M, N, K = 597, 11008, 512
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=77)
    C1, _ = run("bf16", A, B)
    C2, _ = run("bf16", A, B)
    assert np.array_equal(C1, C2)


def test_degenerate_shapes():
    import torch
    from parity import alloc_c, dev_bf16, guard_untouched
    A = dev_bf16(np.ones((4, 32), np.uint16) * 0x3F80)
    B = dev_bf16(np.ones((16, 32), np.uint16) * 0x3F80)
    Bs = dg.shuffle_b(B)
    buf, C = alloc_c(0, 16)
    dg.gemm_bf16(A[:0], Bs, 16, out=C)
    torch.cuda.synchronize()
    assert guard_untouched(buf, 0, 16)
    # K = 0: empty sum, C := 0
    buf, C = alloc_c(4, 16)
    dg.gemm_bf16(A[:, :0], Bs, 16, out=C)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert (h[:4, :16] == 0).all() and guard_untouched(buf, 4, 16)


def test_hip_errors_surface():
    import torch
    A = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    Bs = torch.zeros(dg.shuffle_b_bytes(16, 32), dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_bf16(A, Bs, 16, tile=dg.tiled(48, 64))
    assert e.value.code == dg.GEMM_ERR_UNSUPPORTED
