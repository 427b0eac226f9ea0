"""Pins for the oracle's GEMM (CPU only).

Each test ties the fp64 triple loop to something other than itself: products
worked by hand, identity and permutation matrices (closed forms), an exact
int64 brute force on small-integer inputs, an independent float64 library
matmul, and the multiply-add count (flops = 2*M*N*K, "GEMM Optimization Guide"
page, section 8.1).  A dropped term, a swapped index, a transposed operand, a
wrong leading dimension or a wrong scale fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import datagen
import oracle


def _bits(x):
    return oracle.bf16_from_f64(np.asarray(x, np.float64))


def test_hand_worked_products(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "gemm_small.json")))["cases"]
    for c in cases:
        A = _bits(c["A"])
        B = _bits(c["B"])
        C = oracle.gemm_bf16(A, B, threads=1)
        np.testing.assert_array_equal(C, np.array(c["C"], np.float64), err_msg=c["name"])
        if "not_C" in c:
            assert not np.array_equal(C, np.array(c["not_C"], np.float64))
        # the e4m3 path on the same small integers (all exact e4m3 values)
        Ae = oracle.e4m3_from_f64(np.array(c["A"], np.float64))
        Be = oracle.e4m3_from_f64(np.array(c["B"], np.float64))
        Ce = oracle.gemm_e4m3(Ae, Be, 1.0, 1.0, threads=1)
        np.testing.assert_array_equal(Ce, np.array(c["C"], np.float64), err_msg=c["name"])


@pytest.mark.parametrize("M,K", [(5, 7), (33, 64), (3, 1)])
def test_identity(M, K):
    A = datagen.to_bf16_bits(datagen.uniform(11, (M, K)))
    eye = _bits(np.eye(K))
    C = oracle.gemm_bf16(A, eye)
    np.testing.assert_array_equal(C, oracle.bf16_to_f64(A))


def test_permutation():
    rng = np.random.default_rng(5)
    M, K = 9, 23
    perm = rng.permutation(K)
    A = datagen.to_bf16_bits(datagen.normal(12, (M, K)))
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0          # B[j][k] = 1 iff k == perm[j]
    C = oracle.gemm_bf16(A, _bits(P))
    np.testing.assert_array_equal(C, oracle.bf16_to_f64(A)[:, perm])


@pytest.mark.parametrize("M,N,K", [(7, 5, 3), (64, 48, 128), (17, 33, 96)])
def test_int64_brute_force(M, N, K):
    Ai = datagen.small_int(21, (M, K)).astype(np.int64)
    Bi = datagen.small_int(22, (N, K)).astype(np.int64)
    exact = np.zeros((M, N), np.int64)
    for m in range(M):
        for n in range(N):
            exact[m, n] = int(np.dot(Ai[m], Bi[n]))
    C = oracle.gemm_bf16(_bits(Ai), _bits(Bi))
    np.testing.assert_array_equal(C, exact.astype(np.float64))
    # scaled e4m3 variant with power-of-two scales stays exact
    Ae = oracle.e4m3_from_f64(Ai.astype(np.float64))
    Be = oracle.e4m3_from_f64(Bi.astype(np.float64))
    Ce = oracle.gemm_e4m3(Ae, Be, 2.0 ** -3, 2.0 ** 2)
    np.testing.assert_array_equal(Ce, exact.astype(np.float64) * 0.5)


def test_library_matmul_general_inputs():
    M, N, K = 40, 56, 200
    A = datagen.to_bf16_bits(datagen.normal(31, (M, K)))
    B = datagen.to_bf16_bits(datagen.normal(32, (N, K), 0.02))
    C = oracle.gemm_bf16(A, B)
    ref = (torch.from_numpy(oracle.bf16_to_f64(A)) @ torch.from_numpy(oracle.bf16_to_f64(B)).T).numpy()
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-14)
    # the decoded values agree with torch's own bf16 decoding
    tA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(tA, oracle.bf16_to_f64(A))


def test_e4m3_scaled_against_library():
    M, N, K = 16, 24, 128
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=77)
    C = oracle.gemm_e4m3(A, B, sa, sb)
    dA = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float64)
    dB = torch.from_numpy(B).view(torch.float8_e4m3fn).to(torch.float64)
    ref = ((dA @ dB.T) * float(np.float32(sa)) * float(np.float32(sb))).numpy()
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12)


def test_multiply_add_count():
    for (M, N, K) in [(3, 4, 5), (1, 11, 64), (8, 8, 8)]:
        _, macs = oracle.gemm_bf16(np.zeros((M, K), np.uint16), np.zeros((N, K), np.uint16),
                                   return_macs=True)
        assert macs == M * N * K
        assert 2 * macs == 2 * M * N * K
    _, macs = oracle.gemm_e4m3(np.zeros((6, 9), np.uint8), np.zeros((5, 9), np.uint8), 1.0, 1.0,
                               return_macs=True)
    assert macs == 6 * 5 * 9


def test_points_match_full_product():
    M, N, K = 21, 19, 64
    A = datagen.to_bf16_bits(datagen.uniform(41, (M, K)))
    B = datagen.to_bf16_bits(datagen.uniform(42, (N, K)))
    C = oracle.gemm_bf16(A, B)
    ms = np.array([0, 20, 7, 3, 20])
    ns = np.array([0, 18, 11, 0, 0])
    np.testing.assert_array_equal(oracle.gemm_points(oracle.ORC_BF16, A, B, ms, ns), C[ms, ns])


def test_points_e4m3_scaled_match_full_product():
    """The per-point path on e4m3 codes with the product of the two dequant
    scales, as the full-size parity checks call it, against the full product
    (which applies the scales one after the other): equal to within one
    rounding of the scale product; exactly equal with power-of-two scales."""
    M, N, K = 23, 17, 192
    A, B, sa, sb = datagen.make_e4m3_pair(M, N, K, config=91)
    C = oracle.gemm_e4m3(A, B, sa, sb)
    ms = np.array([0, 22, 5, 11, 22, 0])
    ns = np.array([0, 16, 3, 16, 0, 9])
    pts = oracle.gemm_points(oracle.ORC_E4M3, A, B, ms, ns,
                             float(np.float32(sa)) * float(np.float32(sb)))
    np.testing.assert_allclose(pts, C[ms, ns], rtol=4 * 2.0 ** -53, atol=0)
    C2 = oracle.gemm_e4m3(A, B, 2.0 ** -3, 2.0 ** 2)
    pts2 = oracle.gemm_points(oracle.ORC_E4M3, A, B, ms, ns, 2.0 ** -3 * 2.0 ** 2)
    np.testing.assert_array_equal(pts2, C2[ms, ns])
    # and the scale really is applied: unscaled points differ by sa * sb
    raw = oracle.gemm_points(oracle.ORC_E4M3, A, B, ms, ns, 1.0)
    np.testing.assert_allclose(raw * float(np.float32(sa)) * float(np.float32(sb)), C[ms, ns],
                               rtol=4 * 2.0 ** -53, atol=0)


def test_threads_do_not_change_result():
    M, N, K = 37, 29, 96
    A = datagen.to_bf16_bits(datagen.normal(51, (M, K)))
    B = datagen.to_bf16_bits(datagen.normal(52, (N, K)))
    np.testing.assert_array_equal(oracle.gemm_bf16(A, B, threads=1), oracle.gemm_bf16(A, B, threads=8))


def test_degenerate_shapes():
    C = oracle.gemm_bf16(np.zeros((3, 0), np.uint16), np.zeros((4, 0), np.uint16))
    np.testing.assert_array_equal(C, np.zeros((3, 4)))       # empty sum
    C = oracle.gemm_bf16(np.zeros((0, 8), np.uint16), np.zeros((4, 8), np.uint16))
    assert C.shape == (0, 4)
