"""Pins of the oracle's transpose and transposed-source preshuffle (oracle.c
orc_transpose; oracle.shuffle_b_t = orc_shuffle_b of orc_transpose).

- A hand-worked 2 x 3 transpose, and transposing twice is the identity.
- Brute force from the layout formula on tiny shapes: byte j of the 16-byte
  unit (n0, k0, g, nl) of shuffle_b_t(Bt) is byte j of element
  B[16 n0 + nl][kb k0 + kp g + j / e] with B[n][k] = Bt[k][n], zero past N
  or K ("GEMM Optimization Guide" page, section 12.1, read in bytes).
- The backward identities on small integers: dX = dY W and dW = dY^T X
  computed through the oracle's C = A B^T equal numpy's integer matmuls.
"""
import numpy as np
import pytest

import oracle


def test_transpose_hand_worked():
    X = np.array([[1, 2, 3], [4, 5, 6]], np.uint16)
    assert np.array_equal(oracle.transpose(X), [[1, 4], [2, 5], [3, 6]])
    Y = np.arange(7 * 13, dtype=np.uint8).reshape(7, 13)
    assert np.array_equal(oracle.transpose(oracle.transpose(Y)), Y)


@pytest.mark.parametrize("e", [1, 2])
@pytest.mark.parametrize("N,K", [(16, 64), (17, 64), (31, 128), (48, 192), (5, 64)])
def test_shuffle_b_t_brute_force(N, K, e):
    rng = np.random.default_rng(N * K + e)
    dt = np.uint8 if e == 1 else np.uint16
    Bt = rng.integers(1, 2 ** (8 * e), size=(K, N), dtype=np.int64).astype(dt)   # no zeros
    Bs = oracle.shuffle_b_t(Bt, e)
    kp, KB = 16 // e, -(-K * e // 64)
    raw = Bt.view(np.uint8).reshape(K, N, e)
    nblk = -(-N // 16)
    assert Bs.size == nblk * 16 * KB * 64
    for n0 in range(nblk):
        for k0 in range(KB):
            for g in range(4):
                for nl in range(16):
                    u = ((n0 * KB + k0) * 4 + g) * 16 + nl
                    unit = Bs[u * 16:(u + 1) * 16]
                    n = 16 * n0 + nl
                    for j in range(16):
                        k = (64 // e) * k0 + kp * g + j // e
                        want = raw[k, n, j % e] if (n < N and k < K) else 0
                        assert unit[j] == want, (n0, k0, g, nl, j)


def test_backward_identities_small():
    rng = np.random.default_rng(3)
    M, N_out, K_in = 7, 5, 9
    dY = rng.integers(-4, 5, (M, N_out)).astype(np.float64)
    W = rng.integers(-4, 5, (N_out, K_in)).astype(np.float64)
    X = rng.integers(-4, 5, (M, K_in)).astype(np.float64)
    b = oracle.bf16_from_f64
    # dX = dY W: C = A B^T with A = dY, B = W^T
    dX = oracle.gemm_bf16(b(dY), oracle.transpose(b(W)))
    assert np.array_equal(dX, dY @ W)
    # dW = dY^T X: A = dY^T, B = X^T
    dW = oracle.gemm_bf16(oracle.transpose(b(dY)), oracle.transpose(b(X)))
    assert np.array_equal(dW, dY.T @ X)
