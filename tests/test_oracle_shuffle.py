"""Pins for the oracle's B preshuffle reference (CPU only).

The layout is the "GEMM Optimization Guide" page, sections 1.4 and 12.1, read
in bytes: (N/16, K/kb, 4, 16, kpack) with kpack = 16 bytes (one 16-byte load
per lane), "16" = the 16 lanes that hold the 16 columns of one MFMA block and
"4" = the lane group; padded rows are zero.  The pins are independent of the
index formula: hand-listed entries of a tiny case, bijectivity and zero-fill
counts, the inverse, and the property the layout exists for: every 64-lane
chunk of 16 bytes per lane is exactly one block of 16 columns of B, lane l
holding column l % 16 and the (l // 16)-th kpack of K, so a consumer that
walks the chunks that way reproduces C = A * B^T.
"""
import itertools

import numpy as np
import pytest

import datagen
import oracle


def test_hand_listed_entries_bf16():
    # B bits = 256*n + k (values are opaque to a byte permutation)
    N, K = 16, 64
    B = (np.arange(N)[:, None] * 256 + np.arange(K)[None, :]).astype(np.uint16)
    Bs = oracle.shuffle_b(B, 2).view(np.uint16)
    # lane 0 (column 0, first kpack): k = 0..7 of row 0
    assert Bs[0:8].tolist() == list(range(0, 8))
    # lane 1 (column 1, first kpack): k = 0..7 of row 1
    assert Bs[8:16].tolist() == [256 + k for k in range(8)]
    # lane 16 (column 0, second kpack): k = 8..15 of row 0
    assert Bs[128:136].tolist() == list(range(8, 16))
    # lane 63 (column 15, fourth kpack): k = 24..31 of row 15
    assert Bs[504:512].tolist() == [15 * 256 + k for k in range(24, 32)]
    # next 1 KiB chunk: the same 16 columns, k = 32..63
    assert Bs[512:520].tolist() == list(range(32, 40))
    assert Bs.size == N * K


def test_hand_listed_entries_fp8():
    N, K = 32, 128
    B = ((np.arange(N)[:, None] * 7 + np.arange(K)[None, :]) % 251).astype(np.uint8)
    Bs = oracle.shuffle_b(B, 1)
    # (N/16, K/64, 4, 16, 16): lane l of chunk (n0, k0) holds
    # B[16*n0 + l%16][64*k0 + 16*(l//16) + 0..15]
    assert Bs[0:16].tolist() == B[0, 0:16].tolist()
    assert Bs[16:32].tolist() == B[1, 0:16].tolist()
    assert Bs[256:272].tolist() == B[0, 16:32].tolist()
    assert Bs[1024:1040].tolist() == B[0, 64:80].tolist()          # (n0=0, k0=1)
    assert Bs[2048:2064].tolist() == B[16, 0:16].tolist()          # (n0=1, k0=0)
    assert Bs.reshape(N // 16, K // 64, 4, 16, 16).shape == (2, 2, 4, 16, 16)


@pytest.mark.parametrize("N,K,e", list(itertools.product([16, 17, 31, 48], [64, 128], [1, 2]))
                         + [(5, 48, 2), (1, 16, 2), (33, 80, 2)])
def test_bijection_zero_fill_and_inverse(N, K, e):
    kb = 64 // e
    rng = np.random.default_rng(N * 1000 + K + e)
    dt = np.uint16 if e == 2 else np.uint8
    # distinct non-zero "ids" so every source element is traceable
    ids = (np.arange(N * K) + 1).reshape(N, K)
    if e == 1:
        assert N * K < 2 ** 32
    Bs_ids = []
    # shuffle the id array byte-plane by byte-plane through a wide type
    B32 = ids.astype(np.uint32)
    for plane in range(4 // e):
        part = ((B32 >> (8 * e * plane)) & ((1 << (8 * e)) - 1)).astype(dt)
        Bs_ids.append(oracle.shuffle_b(part, e).view(dt).astype(np.uint32) << (8 * e * plane))
    flat = np.bitwise_or.reduce(np.stack(Bs_ids), axis=0)
    nblk = (N + 15) // 16
    kpad = (K + kb - 1) // kb * kb
    assert flat.size == nblk * 16 * kpad
    nz = flat[flat != 0]
    assert nz.size == N * K                                    # every element once
    assert np.array_equal(np.sort(nz), np.arange(1, N * K + 1))
    assert (flat == 0).sum() == nblk * 16 * kpad - N * K       # zero fill count
    B = rng.integers(0, 2 ** (8 * e), size=(N, K)).astype(dt)
    Bs = oracle.shuffle_b(B, e)
    np.testing.assert_array_equal(oracle.unshuffle_b(Bs, N, K, e), B)


@pytest.mark.parametrize("M,N,K,e", [(3, 16, 64, 2), (5, 40, 96, 2), (4, 33, 128, 1), (2, 16, 64, 1)])
def test_lane_consumer_reproduces_product(M, N, K, e):
    """Walk the shuffled bytes as 64-lane chunks of 16 bytes per lane: lane l
    supplies column 16*n0 + l%16 and the (l//16)-th kpack of K block k0; the
    same lane reads the matching kpack of each A row.  Summing the lane
    products must give the plain GEMM."""
    kp = 16 // e
    kb = 4 * kp
    if e == 2:
        A = datagen.to_bf16_bits(datagen.small_int(61, (M, K)))
        B = datagen.to_bf16_bits(datagen.small_int(62, (N, K)))
        dec = oracle.bf16_to_f64
        view = np.uint16
    else:
        A = oracle.e4m3_from_f64(datagen.small_int(61, (M, K)))
        B = oracle.e4m3_from_f64(datagen.small_int(62, (N, K)))
        dec = oracle.e4m3_to_f64
        view = np.uint8
    Bs = oracle.shuffle_b(B, e).view(view)
    nblk = (N + 15) // 16
    kblk = (K + kb - 1) // kb
    chunks = dec(Bs).reshape(nblk, kblk, 64, kp)          # (n0, k0, lane, j)
    Ad = np.zeros((M, kblk * kb))
    Ad[:, :K] = dec(A)
    C = np.zeros((M, nblk * 16))
    for n0 in range(nblk):
        for k0 in range(kblk):
            for lane in range(64):
                col = 16 * n0 + lane % 16
                ks = k0 * kb + kp * (lane // 16) + np.arange(kp)
                C[:, col] += Ad[:, ks] @ chunks[n0, k0, lane]
    ref = oracle.gemm_bf16(A, B) if e == 2 else oracle.gemm_e4m3(A, B, 1.0, 1.0)
    np.testing.assert_array_equal(C[:, :N], ref)
    assert (C[:, N:] == 0).all()
