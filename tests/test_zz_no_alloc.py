"""gemm_bf16_noalloc (split-K partials in the library's fixed scratch array)
against gemm_bf16_ws with a caller workspace of the same size, through the C
ABI: two calls in a row, the second on a smaller input, each bitwise equal
to the workspace entry point and, on small-integer inputs, to the oracle.
A forced split-K tile whose partials exceed the scratch is refused before
any launch."""
import gc
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
import oracle
from parity import check_exact, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

SCRATCH = dg.NOALLOC_SCRATCH_BYTES


def _both(M, N, K, cfg, tile=None):
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=cfg)
    Ad, Bs = dev_bf16(A), dg.shuffle_b(dev_bf16(B))
    c_ws = torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    c_na = torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ws = torch.full((SCRATCH,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-poisoned
    dg.gemm_bf16(Ad, Bs, N, out=c_ws, tile=tile, workspace=ws)
    torch.cuda.synchronize()
    # torch's allocator count must not change across the call; the garbage
    # collector is kept from freeing earlier tests' tensors meanwhile
    gc.collect()
    gc.disable()
    try:
        before = torch.cuda.memory_allocated()
        dg.gemm_bf16_noalloc(Ad, Bs, N, out=c_na, tile=tile)
        torch.cuda.synchronize()
        after = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    assert after == before
    return A, B, host_bits(c_ws), host_bits(c_na)


@pytest.mark.parametrize("first,second", [
    ((597, 1376, 4096, 61), (48, 4096, 4096, 43)),     # TP-8 up shard, then M = 48
    ((48, 4096, 4096, 43), (40, 1000, 1024, 7)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for (M, N, K, cfg) in (first, second):
        t = dg.select_tile(M, N, K, "bf16", workspace_bytes=SCRATCH)
        print(f"[noalloc {M}x{N}x{K} tile={t.name}]", flush=True)
        A, B, c_ws, c_na = _both(M, N, K, cfg)
        assert np.array_equal(c_na, c_ws), f"{M}x{N}x{K}: differs from gemm_bf16_ws"
        check_exact(c_na, oracle.gemm_bf16(A, B), f"noalloc {M}x{N}x{K}")


def test_noalloc_forced_split_tiles():
    # forced split-K tiles that fit, in a row, the second smaller
    for (M, N, K, tile) in ((300, 270, 2048, dg.with_split(dg.tiled(64, 64), 8)),
                            (64, 200, 1024, dg.with_split(dg.tiled(64, 64), 4))):
        print(f"[noalloc forced {M}x{N}x{K} {tile.name}]", flush=True)
        A, B, c_ws, c_na = _both(M, N, K, 11 + M, tile)
        assert np.array_equal(c_na, c_ws)
        check_exact(c_na, oracle.gemm_bf16(A, B), f"noalloc forced {tile.name}")


def test_noalloc_refuses_partials_beyond_the_scratch():
    M, N, K = 4096, 4096, 4096
    tile = dg.with_split(dg.tiled(128, 128), 16)
    assert dg.workspace_bytes(M, N, K, "bf16", tile) > SCRATCH
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    Bs = torch.zeros(dg.shuffle_b_bytes(N, K), dtype=torch.uint8, device="cuda")
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_bf16_noalloc(A, Bs, N, out=C, tile=tile)
    assert e.value.code == dg.GEMM_ERR_INVALID_VALUE
    torch.cuda.synchronize()
