"""Device shuffle_b against the oracle's preshuffle: bit-identical bytes,
including the zero fill past N and past K, for aligned and unaligned row
pitches."""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
import oracle
from parity import dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(16, 64), (17, 48), (31, 16), (48, 128), (11008, 4096),
                                 (50257, 512), (4095, 1024), (1, 32)])
@pytest.mark.parametrize("pad", [0, 8, 3])
def test_shuffle_bf16(N, K, pad):
    if N * K > 5_000_000 and pad:
        pytest.skip("padded pitch covered on the small shapes")
    B = datagen.to_bf16_bits(datagen.uniform(N + K, (N, K)))
    full = np.zeros((N, K + pad), np.uint16)
    full[:, :K] = B + 0
    Bd = dev_bf16(full)[:, :K]
    Bs = dg.shuffle_b(Bd)
    torch.cuda.synchronize()
    got = Bs.cpu().numpy()
    np.testing.assert_array_equal(got, oracle.shuffle_b(B, 2))


@pytest.mark.parametrize("N,K", [(16, 64), (33, 128), (4096, 4096), (100, 320)])
@pytest.mark.parametrize("pad", [0, 16, 5])
def test_shuffle_fp8(N, K, pad):
    codes, _ = datagen.to_e4m3(datagen.normal(N * 3 + K, (N, K)))
    full = np.zeros((N, K + pad), np.uint8)
    full[:, :K] = codes
    Bd = dev_u8(full)[:, :K]
    Bs = dg.shuffle_b(Bd, dtype="fp8")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Bs.cpu().numpy(), oracle.shuffle_b(codes, 1))
