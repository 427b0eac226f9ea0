"""Fused epilogue on the GPU against the oracle (C ABI, *_ex entry points).

C[m][n] = bf16( act( acc * scale_m[m] * scale_n[n] + bias[n] ) * mul[m][n] )
(for e4m3, acc already times the per-tensor scales), compared with the
oracle's fp64 epilogue on its fp64 product.

Bars:
- bit-exact where the answer is unique: small-integer operands, bias and
  multiplier, power-of-two scales, no activation or ReLU (every intermediate
  is an integer times a power of two well inside fp32);
- otherwise the relative Frobenius bound of parity.py and a per-element bound:
  the fp32 accumulation bound of parity.py carried through the scales, the
  activation's slope (at most 1.2 for SiLU and both GELU forms) and |mul|,
  plus the fp32 activation's own error and the bf16 rounding of the result.
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
import oracle
from parity import REL_FRO, abs_bits, alloc_c, dev_bf16, dev_u8, guard_untouched, host_bits

pytestmark = pytest.mark.gpu

ACTS = {"none": oracle.ACT_NONE, "relu": oracle.ACT_RELU, "silu": oracle.ACT_SILU,
        "gelu_erf": oracle.ACT_GELU_ERF, "gelu_tanh": oracle.ACT_GELU_TANH}


def bf16_bits(x):
    return oracle.bf16_from_f64(np.asarray(x, np.float64))


def make_parts(M, N, exact: bool, seed: int, parts=("scale_m", "scale_n", "bias", "mul")):
    rng = np.random.default_rng(seed)
    d = {}
    if "scale_m" in parts:
        d["scale_m"] = (2.0 ** rng.integers(-2, 3, M) if exact else rng.uniform(0.25, 2.0, M)).astype(np.float32)
    if "scale_n" in parts:
        d["scale_n"] = (2.0 ** rng.integers(-2, 3, N) if exact else rng.uniform(0.25, 2.0, N)).astype(np.float32)
    if "bias" in parts:
        d["bias"] = bf16_bits(rng.integers(-6, 7, N) if exact else rng.normal(0, 2, N))
    if "mul" in parts:
        d["mul"] = bf16_bits(rng.integers(-3, 4, (M, N)) if exact else rng.normal(0, 1, (M, N)))
    return d


def run_epi(dt, A, B, parts, act, tile=None, sa=1.0, sb=1.0, workspace=None, inplace=False,
            ldc=None, col0=0):
    M, K = A.shape
    N = B.shape[0]
    Ad = dev_bf16(A) if dt == "bf16" else dev_u8(A)
    Bd = dev_bf16(B) if dt == "bf16" else dev_u8(B)
    Bs = dg.shuffle_b(Bd, dtype=dt)
    buf, C = alloc_c(M, N, ldc, col0=col0)
    kw = {}
    if "scale_m" in parts:
        kw["scale_m"] = torch.from_numpy(parts["scale_m"]).cuda()
    if "scale_n" in parts:
        kw["scale_n"] = torch.from_numpy(parts["scale_n"]).cuda()
    if "bias" in parts:
        kw["bias"] = dev_bf16(parts["bias"])
    if "mul" in parts:
        if inplace:
            C.copy_(dev_bf16(parts["mul"]))
            kw["mul"] = C
        else:
            kw["mul"] = dev_bf16(parts["mul"])
    print(f"[epilogue {dt} {M}x{N}x{K} tile={tile.name if tile else 'auto'} act={act} "
          f"parts={sorted(parts)} inplace={inplace}]", flush=True)
    if dt == "bf16":
        dg.gemm_bf16(Ad, Bs, N, out=C, tile=tile, workspace=workspace, activation=act, **kw)
    else:
        s_a = torch.tensor([sa], dtype=torch.float32, device="cuda")
        s_b = torch.tensor([sb], dtype=torch.float32, device="cuda")
        dg.gemm_fp8_scaled(Ad, Bs, N, s_a, s_b, out=C, tile=tile, workspace=workspace,
                           activation=act, **kw)
    torch.cuda.synchronize()
    return host_bits(C), guard_untouched(buf, M, N, col0)


def oracle_epi(dt, A, B, parts, act, sa=1.0, sb=1.0):
    prod = oracle.gemm_bf16(A, B) if dt == "bf16" else oracle.gemm_e4m3(A, B, sa, sb)
    return prod, oracle.epilogue(prod, parts.get("scale_m"), parts.get("scale_n"),
                                 parts.get("bias"), ACTS[act], parts.get("mul"))


def check_exact(got, want, what):
    w = oracle.bf16_from_f64(want)
    g = got.copy()
    g[g == 0x8000] = 0
    w[w == 0x8000] = 0
    bad = np.argwhere(g != w)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first {bad[:4].tolist()}"


def check_epi_close(dt, got_bits, want, absprod, K, parts, scale, what):
    got = oracle.bf16_to_f64(got_bits)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = got - want
    fro = np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300)
    assert fro <= REL_FRO[dt], f"{what}: relative Frobenius error {fro:.3e}"
    M, N = want.shape
    sm = np.abs(parts.get("scale_m", np.ones(M, np.float32))).astype(np.float64)[:, None]
    sn = np.abs(parts.get("scale_n", np.ones(N, np.float32))).astype(np.float64)[None, :]
    mul = np.abs(oracle.bf16_to_f64(parts["mul"])) if "mul" in parts else 1.0
    g = (K + 2) * 2.0 ** -24 if dt == "bf16" else 2.0 ** -12 + (K / 128 + 2) * 2.0 ** -24
    acc_err = g * absprod * abs(scale) * sm * sn
    # pre-activation magnitude, for the fp32 evaluation of scale, bias, act
    bias = np.abs(oracle.bf16_to_f64(parts["bias"]))[None, :] if "bias" in parts else 0.0
    pre = absprod * abs(scale) * sm * sn + bias
    bound = 2.0 ** -8 * np.abs(want) + mul * (1.2 * acc_err + 4e-6 * pre + 1e-6) + 1e-30
    viol = np.argwhere(np.abs(err) > bound)
    assert viol.size == 0, f"{what}: {len(viol)} elements out of bound, first {viol[:4].tolist()}"


BF16_TILES = [None, dg.tiled(64, 64), dg.tiled(128, 128, 4, 32), dg.tiled(256, 128, 8),
              dg.tiled_ab(256, 256, 8, 32), dg.tiled_ab(128, 128, 4, 32), dg.tiled_pp(256, 256),
              dg.with_split(dg.tiled(128, 128, 4, 32), 3)]
TILE_IDS = ["auto", "t64x64", "t128x128a32", "t256x128w8", "ab256x256w8a32", "ab128x128a32",
            "pp256x256", "t128x128a32sk3"]


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("tile", BF16_TILES, ids=TILE_IDS)
def test_exact_bf16(tile, act):
    M, N, K = 263, 270, 176
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=31)
    parts = make_parts(M, N, True, 1)
    C, ok = run_epi("bf16", A, B, parts, act, tile)
    assert ok, "guard band written"
    check_exact(C, oracle_epi("bf16", A, B, parts, act)[1], f"{tile} {act}")


@pytest.mark.parametrize("act", ["silu", "gelu_erf", "gelu_tanh", "relu"])
@pytest.mark.parametrize("tile", BF16_TILES, ids=TILE_IDS)
def test_activations_bf16(tile, act):
    M, N, K = 263, 270, 176
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=32)
    parts = make_parts(M, N, False, 2)
    C, ok = run_epi("bf16", A, B, parts, act, tile)
    assert ok
    prod, want = oracle_epi("bf16", A, B, parts, act)
    absprod = oracle.gemm_bf16(abs_bits("bf16", A), abs_bits("bf16", B))
    check_epi_close("bf16", C, want, absprod, K, parts, 1.0, f"{tile} {act}")


@pytest.mark.parametrize("tile", [dg.skinny(16, 16), dg.skinny(48, 32), dg.skinny(16, 16, 8)],
                         ids=lambda t: t.name)
@pytest.mark.parametrize("act", ["relu", "silu"])
def test_skinny(tile, act):
    M, N, K = tile.tile_m - 3, 270, 320
    for exact in (True, False):
        dist = "smallint" if exact else "normal"
        A, B = datagen.make_bf16_pair(M, N, K, dist, dist, config=33)
        parts = make_parts(M, N, exact, 3)
        C, ok = run_epi("bf16", A, B, parts, act if not exact else "relu", tile)
        assert ok
        prod, want = oracle_epi("bf16", A, B, parts, act if not exact else "relu")
        if exact:
            check_exact(C, want, tile.name)
        else:
            absprod = oracle.gemm_bf16(abs_bits("bf16", A), abs_bits("bf16", B))
            check_epi_close("bf16", C, want, absprod, K, parts, 1.0, tile.name)


FP8_TILES = [None, dg.tiled(128, 128, 4, 32), dg.tiled_ab(256, 256, 8, 32),
             dg.tiled_ab(256, 256, 4, 32, stages=4, tile_k=64), dg.tiled_pp(256, 256),
             dg.skinny(32, 16), dg.with_split(dg.tiled(64, 64), 2)]


@pytest.mark.parametrize("tile", FP8_TILES, ids=lambda t: t.name if t else "auto")
def test_fp8_per_token_and_channel_scales(tile):
    M, N, K = (29, 270, 320) if tile is not None and tile.kernel == dg.GEMM_KERNEL_SKINNY \
        else (200, 333, 1088)
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=34, smallint=True)
    parts = make_parts(M, N, True, 4)
    C, ok = run_epi("fp8", A, B, parts, "relu", tile, sa=2.0 ** -3, sb=2.0 ** 2)
    assert ok
    check_exact(C, oracle_epi("fp8", A, B, parts, "relu", 2.0 ** -3, 2.0 ** 2)[1], str(tile))
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=35)
    parts = make_parts(M, N, False, 5, parts=("scale_m", "scale_n", "bias"))
    C, ok = run_epi("fp8", A, B, parts, "gelu_tanh", tile, sa=sa, sb=sb)
    assert ok
    prod, want = oracle_epi("fp8", A, B, parts, "gelu_tanh", sa, sb)
    absprod = oracle.gemm_e4m3(abs_bits("fp8", A), abs_bits("fp8", B), 1.0, 1.0)
    check_epi_close("fp8", C, want, absprod, K, parts, sa * sb, str(tile))


def test_fp8_scales_at_4096_cube_auto_plan():
    """e4m3 4096^3 with per-row and per-column scales and no tile: the plan for
    a plain launch is the 4-wave 256 x 256 rung, which a fused launch replaces
    with the 8-wave one.  Every element against the oracle."""
    M = N = K = 4096
    assert dg.select_tile(M, N, K, "fp8", 256).name == "ab256x256w4a32s4k64"
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=36, smallint=True)
    parts = make_parts(M, N, True, 6, parts=("scale_m", "scale_n"))
    C, ok = run_epi("fp8", A, B, parts, "none", None, sa=2.0 ** -3, sb=2.0 ** 2)
    assert ok
    check_exact(C, oracle_epi("fp8", A, B, parts, "none", 2.0 ** -3, 2.0 ** 2)[1], "auto 4096^3")


@pytest.mark.parametrize("tile", [None, dg.tiled_pp(256, 256), dg.with_split(dg.tiled(64, 64), 2),
                                  dg.skinny(32, 16)], ids=lambda t: t.name if t else "auto")
def test_mul_in_place(tile):
    """SiLU(X W_gate^T) * U written over U (mul is the output itself)."""
    M, N, K = (30, 200, 256) if tile is not None and tile.kernel == dg.GEMM_KERNEL_SKINNY \
        else (150, 300, 256)
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=36)
    parts = make_parts(M, N, True, 6, parts=("mul",))
    C, ok = run_epi("bf16", A, B, parts, "relu", tile, inplace=True)
    assert ok
    check_exact(C, oracle_epi("bf16", A, B, parts, "relu")[1], f"in place {tile}")


def test_k_zero_applies_epilogue_to_zero():
    M, N = 37, 70
    A = np.zeros((M, 0), np.uint16)
    B = np.zeros((N, 0), np.uint16)
    parts = make_parts(M, N, False, 7)
    Ad = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    buf, C = alloc_c(M, N)
    kw = dict(scale_m=torch.from_numpy(parts["scale_m"]).cuda(),
              scale_n=torch.from_numpy(parts["scale_n"]).cuda(), bias=dev_bf16(parts["bias"]),
              mul=dev_bf16(parts["mul"]), activation="gelu_erf")
    Bs = torch.empty(16, dtype=torch.uint8, device="cuda")
    dg.gemm_bf16(Ad, Bs, N, out=C, **kw)
    torch.cuda.synchronize()
    assert guard_untouched(buf, M, N)
    want = oracle.epilogue(np.zeros((M, N)), parts["scale_m"], parts["scale_n"], parts["bias"],
                           oracle.ACT_GELU_ERF, parts["mul"])
    check_epi_close("bf16", host_bits(C), want, np.zeros((M, N)), 0, parts, 1.0, "K=0")
    del A, B


@pytest.mark.parametrize("N", [272, 270], ids=["mul_16B_rows", "mul_2B_rows"])
@pytest.mark.parametrize("tile", [dg.tiled(128, 256, 4, 32), dg.tiled_ab(256, 256, 8, 32),
                                  dg.tiled_pp(256, 256), dg.tiled(64, 64)],
                         ids=lambda t: t.name)
@pytest.mark.parametrize("inplace", [False, True], ids=["mul", "mul_in_place"])
def test_mul_staging_paths(tile, N, inplace):
    """The multiplier goes through the staging area in 16-byte row pieces when
    its base and row pitch allow (N % 8 == 0 here), else element by element."""
    M, K = 300, 192
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=37)
    parts = make_parts(M, N, True, 8, parts=("bias", "mul"))
    C, ok = run_epi("bf16", A, B, parts, "relu", tile, inplace=inplace)
    assert ok
    check_exact(C, oracle_epi("bf16", A, B, parts, "relu")[1], f"{tile.name} N={N}")


@pytest.mark.parametrize("inplace", [False, True], ids=["mul", "mul_in_place"])
def test_epilogue_across_two_launches(inplace):
    """1024 x 50257 x 512 runs as two GEMMs over column ranges (the chosen
    tile's last round would be nearly empty, gemm_plan): the second one's
    bias, column scales and multiplier start at the first's last column."""
    M, N, K = 1024, 50257, 512
    assert dg.plan(M, N, K, "bf16", 256, 0)[1] is not None, "shape no longer splits"
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=212)
    parts = make_parts(M, N, True, 13)
    C, ok = run_epi("bf16", A, B, parts, "relu", None, inplace=inplace)
    assert ok
    check_exact(C, oracle_epi("bf16", A, B, parts, "relu")[1], "epilogue across two launches")


@pytest.mark.parametrize("inplace", [False, True], ids=["mul", "mul_in_place"])
def test_epilogue_across_two_launches_over_rows(inplace):
    """8704 x 2048 x 1024 runs as two GEMMs over row ranges (gemm_plan's row
    split, rows [0, 8192) and the rest): the second one's row scales and
    multiplier start at the first's last row."""
    M, N, K = 8704, 2048, 1024
    plan = dg.plan(M, N, K, "bf16", 256, 0)
    assert plan[1] is not None and plan[3] == 8192, "shape no longer splits by rows"
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=216)
    parts = make_parts(M, N, True, 14)
    C, ok = run_epi("bf16", A, B, parts, "relu", None, inplace=inplace)
    assert ok
    check_exact(C, oracle_epi("bf16", A, B, parts, "relu")[1], "epilogue across two launches over rows")


@pytest.mark.parametrize("tile", [dg.tiled(128, 256, 4, 32), dg.tiled_ab(256, 256, 8, 32),
                                  dg.tiled_pp(256, 256), dg.tiled(64, 64)],
                         ids=lambda t: t.name)
@pytest.mark.parametrize("inplace", [False, True], ids=["mul", "mul_in_place"])
def test_mul_with_odd_c_pitch(tile, inplace):
    """C rows at odd 2-byte phases: the multiplier is staged at each row's
    phase, element by element, also when its own rows are 16-byte aligned
    (a separate multiplier with N % 8 == 0), and when it is C itself."""
    M, N, K = 300, 272, 192
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=38)
    parts = make_parts(M, N, True, 9)
    C, ok = run_epi("bf16", A, B, parts, "relu", tile, inplace=inplace, ldc=N + 5, col0=3)
    assert ok
    check_exact(C, oracle_epi("bf16", A, B, parts, "relu")[1], f"{tile.name} odd pitch")
