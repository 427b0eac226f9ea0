"""The largest sizes the C ABI accepts, on the GPU against the oracle.

Buffer descriptors hold 32-bit byte counts, so the ABI accepts K up to 1 MiB
of bytes per row (bf16 K = 2^19, e4m3 K = 2^20) and row pitches up to 4 MiB
(lda * e, ldc * 2), and rejects more (tests/test_abi.py).  Here each limit is
run, on the skinny kernel, a tiled rung and a split-K rung: small-integer
inputs, so the outputs are bit-exact (every partial sum is an integer below
2^24).  One past each limit is GEMM_ERR_UNSUPPORTED.
"""
import functools

import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
from parity import (alloc_c, check_exact, dev_bf16, dev_u8, guard_untouched, host_bits,
                    oracle_full)

pytestmark = pytest.mark.gpu

K_BF16_MAX = 1 << 19     # 1 MiB of bf16 per row
K_FP8_MAX = 1 << 20      # 1 MiB of e4m3 per row
PITCH_MAX = 1 << 21      # bf16 elements in a 4 MiB row


@functools.lru_cache(maxsize=1)
def bf16_max_k():
    return datagen.make_bf16_pair(70, 24, K_BF16_MAX, "smallint", "smallint", config=201)


@functools.lru_cache(maxsize=1)
def fp8_max_k():
    A, B, _, _ = datagen.make_e4m3_pair(70, 24, K_FP8_MAX, config=202, smallint=True)
    return A, B


CASES = [("skinny", 16, dg.skinny(16, 16)), ("tiled", 70, dg.tiled(64, 64)),
         ("split_k", 70, dg.with_split(dg.tiled(64, 64), 8))]


@pytest.mark.parametrize("name,M,tile", CASES, ids=[c[0] for c in CASES])
def test_bf16_largest_k(name, M, tile):
    A, B = bf16_max_k()
    A = np.ascontiguousarray(A[:M])
    N, K = B.shape
    print(f"[bf16 K={K} M={M} N={N} {tile.name}]", flush=True)
    Ad, Bs = dev_bf16(A), dg.shuffle_b(dev_bf16(B))
    buf, C = alloc_c(M, N)
    ws = None
    if tile.k_split > 1 and tile.kernel != dg.GEMM_KERNEL_SKINNY:
        ws = torch.full((dg.workspace_bytes(M, N, K, "bf16", tile),), 0xFF, dtype=torch.uint8,
                        device="cuda")
    dg.gemm_bf16(Ad, Bs, N, out=C, tile=tile, workspace=ws)
    torch.cuda.synchronize()
    assert guard_untouched(buf, M, N)
    check_exact(host_bits(C), oracle_full("bf16", A, B), f"bf16 K=2^19 {name}")


@pytest.mark.parametrize("name,M,tile", CASES, ids=[c[0] for c in CASES])
def test_fp8_largest_k(name, M, tile):
    A, B = fp8_max_k()
    A = np.ascontiguousarray(A[:M])
    N, K = B.shape
    print(f"[fp8 K={K} M={M} N={N} {tile.name}]", flush=True)
    Ad, Bs = dev_u8(A), dg.shuffle_b(dev_u8(B), dtype="fp8")
    sa = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    sb = torch.tensor([4.0], dtype=torch.float32, device="cuda")
    buf, C = alloc_c(M, N)
    ws = None
    if tile.k_split > 1 and tile.kernel != dg.GEMM_KERNEL_SKINNY:
        ws = torch.full((dg.workspace_bytes(M, N, K, "fp8", tile),), 0xFF, dtype=torch.uint8,
                        device="cuda")
    dg.gemm_fp8_scaled(Ad, Bs, N, sa, sb, out=C, tile=tile, workspace=ws)
    torch.cuda.synchronize()
    assert guard_untouched(buf, M, N)
    check_exact(host_bits(C), oracle_full("fp8", A, B, 0.5, 4.0), f"fp8 K=2^20 {name}")


def test_k_past_limit_unsupported():
    M, N = 16, 32
    A = torch.zeros((M, K_BF16_MAX + 16), dtype=torch.bfloat16, device="cuda")
    Bs = torch.zeros(dg.shuffle_b_bytes(N, K_BF16_MAX + 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.GemmError, match="UNSUPPORTED"):
        dg.gemm_bf16(A, Bs, N)


@pytest.mark.parametrize("tile", [None, dg.tiled_ab(256, 256, 8, 32), dg.skinny(64, 16)],
                         ids=["auto", "ab256x256w8a32", "skinny64x16"])
def test_largest_pitches(tile):
    """A with lda = 2^21 elements and C with ldc = 2^21 (4 MiB rows, the
    limit), several row tiles and a ragged edge."""
    M = 64 if tile is not None and tile.kernel == dg.GEMM_KERNEL_SKINNY else 300
    N, K = 270, 256
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=203)
    Abuf = torch.zeros((M, PITCH_MAX), dtype=torch.bfloat16, device="cuda")
    Abuf[:, :K] = dev_bf16(A)
    Bs = dg.shuffle_b(dev_bf16(B))
    buf, C = alloc_c(M, N, ldc=PITCH_MAX, col0=5)
    print(f"[pitches lda=ldc=2^21 M={M} {tile.name if tile else 'auto'}]", flush=True)
    dg.gemm_bf16(Abuf[:, :K], Bs, N, out=C, tile=tile)
    torch.cuda.synchronize()
    assert guard_untouched(buf, M, N, col0=5)
    check_exact(host_bits(C), oracle_full("bf16", A, B), "lda = ldc = 2^21")
    del buf, Abuf
    # one element more in either pitch is rejected before any launch
    Abig = torch.zeros((2, PITCH_MAX + 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.GemmError, match="UNSUPPORTED"):
        dg.gemm_bf16(Abig[:, :K], Bs, N)
