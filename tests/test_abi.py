"""The C-ABI library on the host (CPU only): it loads, exports every entry
point include/densegemm.h declares, rejects bad arguments before touching the
device, and its pure-host parts (select_tile, shuffle_b_bytes) agree with the
oracle's definitions.  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_gemm_linear_amd as dg
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "densegemm.h")

CONFIG_SHAPES = [(128, 256, 128), (4096, 4096, 4096), (597, 11008, 4096), (1, 11008, 4096),
                 (8, 4096, 4096), (48, 4096, 4096), (3402, 4096, 1024), (1024, 50257, 512),
                 (2048, 11007, 1024), (4095, 4095, 1024), (528, 528, 1024), (32, 4096, 4096)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)) - {"if"})


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(dg.EXPORTS)
    raw = ctypes.CDLL(dg.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings():
    assert dg.gemm_status_string(0) == "GEMM_OK"
    assert dg.gemm_status_string(1) == "GEMM_ERR_INVALID_VALUE"
    assert dg.gemm_status_string(2) == "GEMM_ERR_UNSUPPORTED"
    assert dg.gemm_status_string(3) == "GEMM_ERR_HIP"
    assert dg.gemm_status_string(99) == "GEMM_ERR_UNKNOWN"


@pytest.mark.parametrize("N,K,dt,e", [(16, 64, "bf16", 2), (17, 48, "bf16", 2), (11008, 4096, "bf16", 2),
                                      (50257, 512, "bf16", 2), (4096, 4096, "fp8", 1), (33, 128, "fp8", 1),
                                      (0, 64, "bf16", 2), (5, 0, "fp8", 1)])
def test_shuffle_b_bytes_matches_oracle(N, K, dt, e):
    assert dg.shuffle_b_bytes(N, K, dt) == oracle.shuffle_b_bytes(N, K, e)


def test_shuffle_b_bytes_fp8_layout_size():
    # (N/16, K/64, 4, 16, 16) bytes for the fp8 workload
    assert dg.shuffle_b_bytes(4096, 4096, "fp8") == (4096 // 16) * (4096 // 64) * 4 * 16 * 16
    assert dg.shuffle_b_bytes(-1, 64, "bf16") == 0


@pytest.mark.parametrize("M,N,K", CONFIG_SHAPES)
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_select_tile_metrics_match_oracle(M, N, K, dt):
    t = dg.select_tile(M, N, K, dt, num_cus=256)
    tiled_kinds = (dg.GEMM_KERNEL_TILED, dg.GEMM_KERNEL_TILED_AB, dg.GEMM_KERNEL_TILED_PP)
    assert t.kernel in tiled_kinds + (dg.GEMM_KERNEL_SKINNY,)
    if t.kernel in tiled_kinds:
        assert t in dg.ladder_tiles(dt) or any(
            (t.kernel, t.tile_m, t.tile_n, t.waves, t.atom, t.lds_stages, t.tile_k) ==
            (r.kernel, r.tile_m, r.tile_n, r.waves, r.atom, r.lds_stages, r.tile_k)
            for r in dg.ladder_tiles(dt))
        assert dg.tile_check(t, M, dt) == dg.GEMM_OK
        tiles, te, we, de = oracle.dim_eff(M, N, t.tile_m, t.tile_n, 256)
        assert abs(t.tile_eff - te) < 1e-6 and abs(t.wq_eff - we) < 1e-6
        # padding screen: padded output at most 1.25x the real one when any tile passes
        assert 1.0 / t.tile_eff <= 1.25 + 1e-6
    else:
        assert (t.tile_m, t.tile_n, t.k_split) in dg.SKINNY_LADDER
        assert M <= t.tile_m < M + 16
    assert t.predicted_us > 0
    assert dg.select_tile(M, N, K, dt, num_cus=256) == t       # deterministic


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_every_python_rung_is_a_library_rung(dt):
    tiles = dg.ladder_tiles(dt)
    assert len({t.name for t in tiles}) == len(tiles)            # no duplicates
    for t in tiles:
        assert dg.tile_check(t, 1000, dt) == dg.GEMM_OK, t.name
    for tm, tn, w in dg.SKINNY_LADDER:
        assert dg.tile_check(dg.skinny(tm, tn, w), tm, dt) == dg.GEMM_OK
        assert dg.tile_check(dg.skinny(tm, tn, w), tm + 1, dt) == dg.GEMM_ERR_UNSUPPORTED
    assert dg.tile_check(dg.skinny(64, 64, 8), 64, dt) == dg.GEMM_ERR_UNSUPPORTED
    # wildcards: stages / tile_k 0 pick the first matching rung
    assert dg.tile_check(dg.tiled(128, 128), 100, dt) == dg.GEMM_OK
    assert dg.tile_check(dg.tiled_ab(256, 256, 8, 32), 100, dt) == dg.GEMM_OK
    # not rungs
    U = dg.GEMM_ERR_UNSUPPORTED
    assert dg.tile_check(dg.tiled(96, 128), 100, dt) == U
    assert dg.tile_check(dg.tiled(128, 128, 4, 32, stages=7), 100, dt) == U
    assert dg.tile_check(dg.tiled(128, 128, 4, 32, tile_k=48), 100, dt) == U
    assert dg.tile_check(dg.tiled_ab(256, 256, 8, 16, stages=3), 100, dt) == U
    # the 16 x 16-atom 256 x 256 rung has 64-byte k-tiles: bf16 only (an e4m3
    # 16 x 16 x 128 MFMA needs 128 K bytes per k-tile)
    a16 = dg.tiled_ab(256, 256, 8, 16, stages=4, tile_k=32 if dt == "bf16" else 64)
    assert dg.tile_check(a16, 100, dt) == (dg.GEMM_OK if dt == "bf16" else U)
    assert dg.tile_check(dg.Tile(7, 128, 128), 100, dt) == U
    assert dg.lib.gemm_tile_check(None, 1, 0) == dg.GEMM_ERR_INVALID_VALUE


def test_select_tile_routes_small_m_to_skinny():
    for M in (1, 8, 16):
        assert dg.select_tile(M, 11008, 4096, "bf16", 256).kernel == dg.GEMM_KERNEL_SKINNY
    assert dg.select_tile(4096, 4096, 4096, "bf16", 256).kernel in (dg.GEMM_KERNEL_TILED,
                                                                    dg.GEMM_KERNEL_TILED_AB,
                                                                    dg.GEMM_KERNEL_TILED_PP)


def test_select_tile_errors():
    t = dg.GemmTile()
    assert dg.lib.select_tile(-1, 4, 4, 0, 256, ctypes.byref(t)) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.lib.select_tile(4, 4, 4, 7, 256, ctypes.byref(t)) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.lib.select_tile(4, 4, 4, 0, 256, None) == dg.GEMM_ERR_INVALID_VALUE


# Fake device addresses: argument checks must reject before any HIP call.
PA = 0x10000
PB = 0x20000
PC = 0x30000


def _bf16(A, lda, Bs, C, ldc, M, N, K, tile=None):
    return dg.lib.gemm_bf16(A, lda, Bs, C, ldc, M, N, K, tile, None)


def test_gemm_bf16_argument_checks():
    E = dg.GEMM_ERR_INVALID_VALUE
    U = dg.GEMM_ERR_UNSUPPORTED
    assert _bf16(PA, 64, PB, PC, 64, 0, 64, 64) == dg.GEMM_OK        # empty: no launch
    assert _bf16(PA, 64, PB, PC, 64, 64, 0, 64) == dg.GEMM_OK
    assert _bf16(None, 64, None, None, 64, 0, 64, 64) == dg.GEMM_OK
    assert _bf16(PA, 64, PB, PC, 64, -1, 64, 64) == E
    assert _bf16(PA, 64, PB, PC, 64, 64, 64, -16) == E
    assert _bf16(None, 64, PB, PC, 64, 64, 64, 64) == E
    assert _bf16(PA, 64, None, PC, 64, 64, 64, 64) == E
    assert _bf16(PA, 64, PB, None, 64, 64, 64, 64) == E
    assert _bf16(PA, 32, PB, PC, 64, 64, 64, 64) == E                 # lda < K
    assert _bf16(PA, 64, PB, PC, 63, 64, 64, 64) == E                 # ldc < N
    assert _bf16(PA + 8, 64, PB, PC, 64, 64, 64, 64) == E             # A not 16-byte aligned
    assert _bf16(PA, 64, PB + 4, PC, 64, 64, 64, 64) == E             # Bs not 16-byte aligned
    assert _bf16(PA, 68, PB, PC, 64, 64, 64, 64) == E                 # lda*2 % 16 != 0
    assert _bf16(PA, 64, PB, PC + 1, 64, 64, 64, 64) == E             # C odd address
    assert _bf16(PA, 64, PB, PC, 64, 64, 64, 40) == U                 # K % 16 != 0
    assert _bf16(None, 0, None, None, 64, 64, 64, 0) == E              # K = 0 still needs C
    bad = dg.tiled(100, 64).to_c()
    assert _bf16(PA, 64, PB, PC, 64, 64, 64, 64, ctypes.byref(bad)) == U
    bad = dg.tiled(64, 64, 8).to_c()                                     # not a rung
    assert _bf16(PA, 64, PB, PC, 64, 64, 64, 64, ctypes.byref(bad)) == U
    bad = dg.skinny(16, 16).to_c()
    assert _bf16(PA, 64, PB, PC, 64, 17, 64, 64, ctypes.byref(bad)) == U   # M > skinny rows


def test_gemm_fp8_argument_checks():
    E = dg.GEMM_ERR_INVALID_VALUE
    U = dg.GEMM_ERR_UNSUPPORTED
    f = dg.lib.gemm_fp8_scaled
    assert f(PA, 128, PB, 0x40000, 0x40010, PC, 64, 0, 64, 128, None, None) == dg.GEMM_OK
    assert f(PA, 128, PB, None, 0x40010, PC, 64, 8, 64, 128, None, None) == E
    assert f(PA, 128, PB, 0x40000, None, PC, 64, 8, 64, 128, None, None) == E
    assert f(PA, 136, PB, 0x40000, 0x40010, PC, 64, 8, 64, 128, None, None) == E   # lda % 16
    assert f(PA, 128, PB, 0x40000, 0x40010, PC, 64, 8, 64, 96, None, None) == U    # K % 64


def test_shuffle_b_argument_checks():
    f = dg.lib.shuffle_b
    assert f(PA, 64, PB, 0, 64, 0, None) == dg.GEMM_OK
    assert f(PA, 64, PB, 16, 0, 0, None) == dg.GEMM_OK
    assert f(None, 64, PB, 16, 64, 0, None) == dg.GEMM_ERR_INVALID_VALUE
    assert f(PA, 32, PB, 16, 64, 0, None) == dg.GEMM_ERR_INVALID_VALUE      # ldb < K
    assert f(PA, 64, PB + 8, 16, 64, 0, None) == dg.GEMM_ERR_INVALID_VALUE  # Bs alignment
    assert f(PA, 64, PB, -16, 64, 0, None) == dg.GEMM_ERR_INVALID_VALUE
    assert f(PA, 96, PB, 16, 96, 1, None) == dg.GEMM_ERR_UNSUPPORTED        # fp8 K % 64
    assert f(PA, 64, PB, 16, 40, 0, None) == dg.GEMM_ERR_UNSUPPORTED        # bf16 K % 16


def test_one_hip_runtime_in_process():
    """The binding must bind to the HIP runtime torch already loaded: exactly
    one libamdhip64 mapped in this process."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().splitlines()
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line and "/" in line}
    assert len(libs) == 1, libs


# ------------------------------------------------------------------ split-K
def _ws_expected(M, N, K, e, ktb, k_split):
    """Workspace of a split-K tile: S slices of ceil(k-tiles / S') k-tiles
    (S' = k_split capped at the k-tile count, S lowered so none is empty),
    each an fp32 plane M x ldw with ldw = N rounded up to 4."""
    nkt = -(-K * e // ktb)
    want = max(1, min(k_split, nkt))
    per = -(-nkt // want)
    S = -(-nkt // per)
    ldw = -(-N // 4) * 4
    return S * M * ldw * 4 if S > 1 else 0


@pytest.mark.parametrize("dt,e", [("bf16", 2), ("fp8", 1)])
def test_workspace_bytes_formula(dt, e):
    rungs = [(dg.tiled(128, 128, 4, 32, 3, 128 // e), 128),
             (dg.tiled_ab(256, 256, 8, 32, 4, 64 // e), 64),
             (dg.tiled_pp(256, 256, 32, 4, 64 // e), 64)]
    for tile, ktb in rungs:
        for M, N in ((263, 270), (597, 1376), (1, 16)):
            for K in (64, 128, 1088, 4096):
                for S in (1, 2, 3, 7, 64):
                    t = dg.with_split(tile, S)
                    got = dg.workspace_bytes(M, N, K, dt, t)
                    assert got == _ws_expected(M, N, K, e, ktb, S), (t.name, M, N, K)
    assert dg.workspace_bytes(16, 64, 4096, dt, dg.skinny(16, 16)) == 0
    assert dg.workspace_bytes(64, 64, 4096, dt, dg.with_split(dg.tiled(64, 64), 65)) == 0
    assert dg.lib.gemm_workspace_bytes(64, 64, 64, 0, None) == 0


def test_select_tile_ws_stays_within_budget():
    shapes = CONFIG_SHAPES + [(597, 1376, 4096), (597, 4096, 1376), (1, 1376, 4096)]
    for M, N, K in shapes:
        for dt in ("bf16", "fp8"):
            if dt == "fp8" and K % 64:
                continue
            plain = dg.select_tile(M, N, K, dt, 256)
            for budget in (1 << 20, 16 << 20, 256 << 20):
                t = dg.select_tile(M, N, K, dt, 256, workspace_bytes=budget)
                assert dg.workspace_bytes(M, N, K, dt, t) <= budget, (M, N, K, dt, budget, t.name)
                assert dg.tile_check(t, M, dt) == dg.GEMM_OK
                if t.k_split > 1 and t.kernel != dg.GEMM_KERNEL_SKINNY:
                    tiles = -(-M // t.tile_m) * -(-N // t.tile_n)
                    assert 2 * tiles <= 256, "split-K only where half the CUs would idle"
                else:
                    assert t == plain
    # an under-filled shape (55 tiles of 128 x 128) is split when memory allows
    t = dg.select_tile(597, 1376, 4096, "bf16", 256, workspace_bytes=256 << 20)
    assert t.k_split > 1


def test_split_k_argument_checks():
    E = dg.GEMM_ERR_INVALID_VALUE
    U = dg.GEMM_ERR_UNSUPPORTED
    split = dg.with_split(dg.tiled(128, 128, 4, 32), 4).to_c()
    need = dg.workspace_bytes(263, 270, 1040, "bf16", dg.Tile.from_c(split))
    assert need > 0
    ws = dg.lib.gemm_bf16_ws

    def call(tile, w, nbytes):
        return ws(PA, 1040, PB, PC, 270, 263, 270, 1040, tile, w, nbytes, None)
    # the plain entry point cannot run a split-K tile
    assert _bf16(PA, 1040, PB, PC, 270, 263, 270, 1040, ctypes.byref(split)) == U
    assert call(ctypes.byref(split), None, 0) == U
    assert call(ctypes.byref(split), 0x40000, need - 4) == E          # too small
    assert call(ctypes.byref(split), 0x40008, need) == E              # not 16-byte aligned
    assert call(None, None, 1024) == E                                # bytes without a pointer
    for k in (-1, 65):
        bad = dg.with_split(dg.tiled(128, 128, 4, 32), k).to_c()
        assert call(ctypes.byref(bad), 0x40000, need) == U
    f = dg.lib.gemm_fp8_scaled_ws
    split8 = dg.with_split(dg.tiled(128, 128, 4, 32), 4).to_c()
    assert f(PA, 1088, PB, 0x50000, 0x50010, PC, 270, 263, 270, 1088, ctypes.byref(split8), None,
             0, None) == U
    assert f(PA, 1088, PB, 0x50000, 0x50010, PC, 270, 263, 270, 1088, ctypes.byref(split8),
             0x40000, 64, None) == E


def test_split_k_rejects_planes_past_32_bit_offsets():
    """(M + 256) * ldw * 4 > 2 GiB: a split-K tile is refused before any launch."""
    t = dg.with_split(dg.tiled(64, 64), 2).to_c()
    N = (1 << 31) // (4 * (1 + 256)) + 64
    assert dg.lib.gemm_bf16_ws(PA, 4096, PB, PC, N, 1, N, 4096, ctypes.byref(t), 0x40000,
                               1 << 40, None) == dg.GEMM_ERR_UNSUPPORTED


def test_epilogue_argument_checks():
    """Bad epilogue arguments are rejected before any launch."""
    E = dg.GEMM_ERR_INVALID_VALUE
    f = dg.lib.gemm_bf16_ex

    def call(epi):
        return f(PA, 64, PB, PC, 64, 64, 64, 64, None, ctypes.byref(epi), None, 0, None)
    e = dg.GemmEpilogue()
    e.activation = 5
    assert call(e) == E
    e.activation = -1
    assert call(e) == E
    e.activation = dg.GEMM_ACT_SILU
    e.bias = 0x50001                      # bf16 bias not 2-byte aligned
    assert call(e) == E
    e.bias = None
    e.scale_m = 0x50002                   # fp32 scales not 4-byte aligned
    assert call(e) == E
    e.scale_m = None
    e.scale_n = 0x50006
    assert call(e) == E
    e.scale_n = None
    e.mul = 0x50000
    e.ld_mul = 63                         # ld_mul < N
    assert call(e) == E
    g = dg.lib.gemm_fp8_scaled_ex
    e.ld_mul = 64
    e.activation = 9
    assert g(PA, 128, PB, 0x40000, 0x40010, PC, 64, 8, 64, 128, None, ctypes.byref(e), None, 0,
             None) == E


def test_transpose_and_shuffle_b_t_argument_checks():
    E = dg.GEMM_ERR_INVALID_VALUE
    U = dg.GEMM_ERR_UNSUPPORTED
    t = dg.lib.transpose_2d
    assert t(PA, 64, PB, 64, 0, 64, 2, None) == dg.GEMM_OK           # empty
    assert t(PA, 64, PB, 64, -1, 64, 2, None) == E
    assert t(PA, 64, PB, 64, 64, 64, 4, None) == E                  # elem_bytes
    assert t(None, 64, PB, 64, 64, 64, 2, None) == E
    assert t(PA, 63, PB, 64, 64, 64, 2, None) == E                  # ld_src < cols
    assert t(PA, 64, PB, 63, 64, 64, 2, None) == E                  # ld_dst < rows
    assert t(PA + 1, 64, PB, 64, 64, 64, 2, None) == E              # misaligned bf16
    assert t(PA, 64, PB, 65536 * 64, 65536 * 64, 64, 1, None) == U  # too many row tiles
    s = dg.lib.shuffle_b_t
    assert s(PA, 64, PB, 64, 0, 0, None) == dg.GEMM_OK
    assert s(PA, 63, PB, 64, 64, 0, None) == E                      # ldbt < N
    assert s(PA, 64, PB + 8, 64, 64, 0, None) == E                  # Bs not 16-byte aligned
    assert s(PA + 1, 64, PB, 64, 64, 0, None) == E                  # Bt not 2-byte aligned
    assert s(PA, 64, PB, 64, 40, 0, None) == U                      # bf16 K % 16
    assert s(PA, 64, PB, 64, 96, 1, None) == U                      # e4m3 K % 64


def test_select_tile_cache_consistent():
    """select_tile keeps its choice per shape; repeated calls, and calls after
    the table has filled (4096 shapes) and been emptied, give the same tile."""
    shapes = [(m, n, k) for m in (1, 48, 597, 4096) for n in (1376, 4095, 11008) for k in (512, 4096)]
    first = {s: dg.select_tile(*s, "bf16", 256) for s in shapes}
    for i in range(4200):                      # more distinct shapes than the table holds
        dg.select_tile(1 + i, 64 + (i % 7), 128, "bf16", 256)
    for s in shapes:
        again = dg.select_tile(*s, "bf16", 256)
        assert again.name == first[s].name and again.predicted_us == first[s].predicted_us, s
    # the workspace size is part of the key
    a = dg.select_tile(48, 4096, 4096, "bf16", 256)
    b = dg.select_tile(48, 4096, 4096, "bf16", 256, workspace_bytes=64 << 20)
    assert a.kernel == dg.GEMM_KERNEL_SKINNY and b.k_split > 1
    assert dg.select_tile(48, 4096, 4096, "bf16", 256).name == a.name


def test_gemm_plan_splits_a_stray_last_round():
    """gemm_plan: lm_head's 788 tiles of 256 x 256 (3 full rounds + 20) run
    as 49152 columns with that tile and 1105 with their own; shapes whose
    rounds are full, or whose rounds are too short to pay a second launch,
    run as one."""
    first, second, n1, m1 = dg.plan(1024, 50257, 512, "bf16", 256, 0)
    assert (first.tile_m, first.tile_n, n1, m1) == (256, 256, 49152, 1024)
    assert second is not None and dg.tile_check(second, 1024, "bf16") == dg.GEMM_OK
    assert first.name == dg.select_tile(1024, 50257, 512, "bf16", 256).name
    for shape in ((4096, 4096, 4096), (512, 50257, 256), (1, 11008, 4096), (597, 11008, 4096)):
        f, s, n, m = dg.plan(*shape, "bf16", 256, 0)
        assert s is None and n == shape[1] and m == shape[0], shape
        assert f.name == dg.select_tile(*shape, "bf16", 256).name
    P = dg.lib.gemm_plan
    t1, t2, n, m = dg.GemmTile(), dg.GemmTile(), ctypes.c_int64(), ctypes.c_int64()
    for bad in ((0, 16, 16, 0, 256), (16, 16, 16, 0, 0), (16, 16, 16, 7, 256)):
        M, N, K, dt, cus = bad
        assert P(M, N, K, dt, cus, 0, ctypes.byref(t1), ctypes.byref(t2), ctypes.byref(n),
                 ctypes.byref(m)) == dg.GEMM_ERR_INVALID_VALUE
    assert P(16, 16, 16, 0, 256, 0, None, ctypes.byref(t2), ctypes.byref(n),
             ctypes.byref(m)) == dg.GEMM_ERR_INVALID_VALUE
    assert P(16, 16, 16, 0, 256, 0, ctypes.byref(t1), ctypes.byref(t2), ctypes.byref(n),
             None) == dg.GEMM_ERR_INVALID_VALUE


def test_gemm_plan_splits_rows_of_a_stray_round():
    """gemm_plan, row split: 10240 x 2048 x 8192 (the GPT-3-XL input gradient)
    has 320 tiles of 256 x 256, one round and a quarter, and no column split
    applies; the rows [0, 8192) make one whole round with the 256 x 256 tile
    and the other 2048 rows run as a second GEMM.  A short K (512) leaves
    8704 x 2048 as one launch, and neither the 4096^3 product nor lm_head
    (a column split) is split by rows."""
    first, second, n1, m1 = dg.plan(10240, 2048, 8192, "bf16", 256, 128 << 20)
    assert (first.tile_m, first.tile_n, n1, m1) == (256, 256, 2048, 8192)
    assert second is not None and dg.tile_check(second, 2048, "bf16") == dg.GEMM_OK
    assert first.name == dg.select_tile(8192, 2048, 8192, "bf16", 256, workspace_bytes=128 << 20).name
    assert second.name == dg.select_tile(2048, 2048, 8192, "bf16", 256, workspace_bytes=128 << 20).name
    for shape, ws in (((8704, 2048, 512), 0), ((4096, 4096, 4096), 0), ((8192, 2048, 10240), 0)):
        f, s, n, m = dg.plan(*shape, "bf16", 256, ws)
        assert s is None and (n, m) == (shape[1], shape[0]), shape
    f, s, n, m = dg.plan(1024, 50257, 512, "bf16", 256, 0)
    assert m == 1024 and n < 50257


def test_select_tile_concurrent_callers_agree():
    """Eight threads query the selector at once (ctypes drops the GIL during
    the call), over more distinct shapes than its table keeps, so lookups,
    inserts and clears interleave; every answer equals the single-threaded one."""
    import threading
    rng = np.random.default_rng(5)
    shapes = [(int(m), int(n), int(k) * 16) for m, n, k in
              zip(rng.integers(1, 5000, 600), rng.integers(16, 60000, 600), rng.integers(1, 512, 600))]
    want = {s: dg.select_tile(*s, "bf16", 256).name for s in shapes}
    errors = []

    def worker(seed):
        r = np.random.default_rng(seed)
        try:
            for j, i in enumerate(r.permutation(len(shapes)).tolist() * 2):
                s = shapes[i]
                got = dg.select_tile(*s, "bf16", 256).name
                if got != want[s]:
                    errors.append((s, got, want[s]))
                # a shape of this thread's own each time: 9600 in all, past the table's 4096
                dg.select_tile(1 + j, 100000 + seed, 64, "bf16", 256)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_binding_rejects_wrong_operand_types_before_any_launch():
    """The binding checks what the C ABI cannot see behind its pointers:
    element types first, so these run without a GPU.  Each mistake raises
    ValueError before anything reaches the library."""
    import torch
    a_bf = torch.zeros((4, 64), dtype=torch.bfloat16)
    a_f8 = torch.zeros((4, 64), dtype=torch.uint8)
    bs = torch.zeros(dg.shuffle_b_bytes(16, 64), dtype=torch.uint8)
    one = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError, match="element type"):
        dg.gemm_bf16(a_f8, bs, 16)                      # e4m3 A to the bf16 GEMM
    with pytest.raises(ValueError, match="element type"):
        dg.gemm_bf16(a_bf.float(), bs, 16)              # fp32 A
    with pytest.raises(ValueError, match="element type"):
        dg.gemm_fp8_scaled(a_bf, bs, 16, one, one)      # bf16 A to the e4m3 GEMM
    with pytest.raises(ValueError, match="scale_a"):
        dg.gemm_fp8_scaled(a_f8, bs, 16, one.double(), one)
    with pytest.raises(ValueError, match="scale_b"):
        dg.gemm_fp8_scaled(a_f8, bs, 16, one, torch.ones(0, dtype=torch.float32))
    with pytest.raises(ValueError, match="scale_a"):
        dg.gemm_fp8_scaled(a_f8, bs, 16, 1.0, one)      # a number, not a tensor
    with pytest.raises(ValueError, match="device"):
        dg.gemm_bf16(a_bf, bs, 16)                      # host A


def test_read_probe_rejects_bad_arguments_before_any_launch():
    """Null pointers, a misaligned buffer and sizes that are zero or not a
    multiple of 16 bytes are refused on the host (the device is never
    reached: this runs without one)."""
    E = dg.GEMM_ERR_INVALID_VALUE
    f = dg.lib.gemm_read_probe
    P = 1 << 20
    assert f(None, 64, P, None) == E
    assert f(P, 64, None, None) == E
    assert f(P + 8, 64, P, None) == E
    assert f(P, 0, P, None) == E
    assert f(P, 72, P, None) == E
    assert f(P, (1 << 40) + 16, P, None) == E
