"""Stream-K on the GPU against the oracle (C ABI, *_ws entry points).

A stream-K launch is a persistent grid of one workgroup per CU; the
(tile, k-tile) units of the stream-K tiles are cut into equal contiguous
ranges, so most tiles are cut between workgroups.  Every workgroup that
holds part of a cut tile writes its fp32 partial to the workspace and counts
itself in; the last to arrive adds the partials in k order and stores C.
The workspace is filled with 0xFF bytes (NaN as fp32) before each call, so a
partial read before it was written poisons the output.

Shapes here have few tiles and many k-tiles, so a tile is cut into many
segments (up to ~30 workgroups for the smallest), and ragged M, N and K.
Bars: bit-exact on small-integer inputs (partial sums are integers below
2^24, exact in any order), the parity.py bounds otherwise, and bitwise
repeatability (the partials are added in a fixed order).
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
from parity import abs_bits, check_close, check_exact, oracle_full, run

pytestmark = pytest.mark.gpu

WS = 128 << 20


def sk_rungs(dt):
    """Every rung with a stream-K instance (outputs of 128 x 128 to 128 x 256)."""
    return [dg.with_stream_k(t) for t in dg.ladder_tiles(dt)
            if t.kernel in (dg.GEMM_KERNEL_TILED, dg.GEMM_KERNEL_TILED_AB)
            and 128 * 128 <= t.tile_m * t.tile_n <= 128 * 256]


def nan_ws():
    return torch.full((WS,), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("tile", sk_rungs("bf16"), ids=lambda t: t.name)
def test_every_stream_k_rung_bf16(tile):
    # 6 or 9 tiles; K = 4176 is 65.25 k-tiles of 128 bytes (a ragged last
    # one), so each tile is cut into tens of segments
    M, N, K = 300, 270, 4176
    need = dg.workspace_bytes(M, N, K, "bf16", tile)
    assert 0 < need <= WS
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=31)
    C, ok = run("bf16", A, B, tile=tile, workspace=nan_ws())
    assert ok, "guard band written"
    check_exact(C, oracle_full("bf16", A, B), tile.name)


@pytest.mark.parametrize("tile", sk_rungs("fp8"), ids=lambda t: t.name)
def test_every_stream_k_rung_fp8(tile):
    M, N, K = 260, 300, 8256
    A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=32, smallint=True)
    C, ok = run("fp8", A, B, tile=tile, sa=2.0 ** -3, sb=4.0, workspace=nan_ws())
    assert ok, "guard band written"
    check_exact(C, oracle_full("fp8", A, B, 2.0 ** -3, 4.0), tile.name)


def test_stream_k_general_inputs_and_repeatable():
    M, N, K = 597, 1376, 4096
    tile = dg.with_stream_k(dg.tiled(128, 256, 4, 32, 3, 64))
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=61, sigma_a=1.0, sigma_b=0.02)
    C1, ok = run("bf16", A, B, tile=tile, workspace=nan_ws())
    assert ok
    check_close("bf16", C1, oracle_full("bf16", A, B),
                oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)), K, what=tile.name)
    C2, _ = run("bf16", A, B, tile=tile, workspace=nan_ws())
    assert np.array_equal(C1, C2), "stream-K result not bitwise repeatable"


def test_stream_k_workspace_reused_across_calls():
    """The tile counters are zeroed by the launch and left zero by the last
    arrivers: back-to-back calls on one workspace, different shapes."""
    ws = nan_ws()
    for (M, N, K, cfg) in ((300, 270, 4160, 41), (129, 500, 2048, 42), (300, 270, 4160, 43)):
        tile = dg.with_stream_k(dg.tiled_ab(128, 128, 4, 32))
        A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=cfg)
        C, ok = run("bf16", A, B, tile=tile, workspace=ws)
        assert ok
        check_exact(C, oracle_full("bf16", A, B), f"{M}x{N}x{K}")


def test_stream_k_refusals():
    A = torch.zeros((300, 4160), dtype=torch.bfloat16, device="cuda")
    Bs = torch.zeros(dg.shuffle_b_bytes(270, 4160), dtype=torch.uint8, device="cuda")
    C = torch.zeros((300, 270), dtype=torch.bfloat16, device="cuda")
    tile = dg.with_stream_k(dg.tiled(128, 256, 4, 32, 3, 64))
    small = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.GemmError) as e:             # workspace too small
        dg.gemm_bf16(A, Bs, 270, out=C, tile=tile, workspace=small)
    assert e.value.code == dg.GEMM_ERR_INVALID_VALUE
    with pytest.raises(dg.GemmError) as e:             # no fused epilogue with stream-K
        dg.gemm_bf16(A, Bs, 270, out=C, tile=tile, workspace=nan_ws(), activation="relu")
    assert e.value.code == dg.GEMM_ERR_UNSUPPORTED
    with pytest.raises(dg.GemmError) as e:             # fewer units than workgroups
        dg.gemm_bf16(A[:, :64], torch.zeros(dg.shuffle_b_bytes(270, 64), dtype=torch.uint8,
                                            device="cuda"), 270, out=C, tile=tile, workspace=nan_ws())
    assert e.value.code == dg.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
