"""Backward GEMMs of a linear layer Y = X W^T on the GPU against the oracle
("TraceLens GEMM analysis" page: the backward pass and the GPT-3-XL table).

- transpose_2d and shuffle_b_t: bit-exact against the oracle (integer and
  byte work), with sentinel-filled destinations to catch stray writes.
- dX = dY W (grad_input: shuffle_b_t(W), then the GEMM) and dW = dY^T X
  (grad_weight: transpose_2d(dY), shuffle_b_t(X), then the GEMM): bit-exact on
  small integers, the parity.py bounds otherwise, and sampled whole rows and
  columns at the GPT-3-XL shapes (10240 tokens, d_model 2048, d_ff 8192).
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
import oracle
from parity import (abs_bits, check_close, check_exact, dev_bf16, dev_u8, host_bits, oracle_full,
                    oracle_lines, sample_lines)

pytestmark = pytest.mark.gpu


def dev(x):
    return dev_bf16(x) if x.dtype == np.uint16 else dev_u8(x)


@pytest.mark.parametrize("e", [1, 2])
@pytest.mark.parametrize("rows,cols,pad_src,pad_dst",
                         [(1, 1, 0, 0), (63, 65, 0, 3), (64, 64, 5, 0), (130, 257, 7, 9),
                          (1000, 37, 0, 0), (37, 1000, 2, 1),
                          # 16-byte pitches: full tiles move in 16-byte pieces, edges by element
                          (64, 64, 0, 0), (256, 320, 0, 0), (200, 136, 8, 8), (136, 200, 24, 56)])
def test_transpose_bit_exact(rows, cols, pad_src, pad_dst, e):
    rng = np.random.default_rng(rows * 7 + cols + e)
    dt = np.uint8 if e == 1 else np.uint16
    src = rng.integers(0, 2 ** (8 * e), size=(rows, cols + pad_src), dtype=np.int64).astype(dt)
    S = dev(src)[:, :cols]
    guard = 3
    sentinel = 0xA5 if e == 1 else 0xA5A5
    buf = torch.full((cols + guard, rows + pad_dst), sentinel if e == 1 else sentinel - 65536,
                     dtype=torch.uint8 if e == 1 else torch.int16, device="cuda")
    D = buf[:cols, :rows]
    print(f"[transpose {rows}x{cols} e={e} pads {pad_src},{pad_dst}]", flush=True)
    dg.transpose(S, out=D)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(dt)
    assert np.array_equal(h[:cols, :rows], oracle.transpose(np.ascontiguousarray(src[:, :cols])))
    h = h.copy()
    h[:cols, :rows] = sentinel
    assert (h == sentinel).all(), "wrote outside the destination view"


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("N,K,pad", [(16, 64, 0), (17, 128, 3), (270, 192, 0), (1377, 512, 8),
                                     (33, 4096, 1), (256, 512, 0), (200, 320, 16)])
def test_shuffle_b_t_bit_exact(N, K, pad, dtype):
    e = 2 if dtype == "bf16" else 1
    rng = np.random.default_rng(N + K + e)
    dt = np.uint8 if e == 1 else np.uint16
    Bt = rng.integers(0, 2 ** (8 * e), size=(K, N + pad), dtype=np.int64).astype(dt)
    print(f"[shuffle_b_t {dtype} N={N} K={K} pad={pad}]", flush=True)
    Bs = dg.shuffle_b_t(dev(Bt)[:, :N], dtype=dtype)
    torch.cuda.synchronize()
    want = oracle.shuffle_b_t(np.ascontiguousarray(Bt[:, :N]), e)
    assert np.array_equal(Bs.cpu().numpy(), want)
    # the same bytes as shuffle_b of the explicit transpose, on the device
    B = np.ascontiguousarray(Bt[:, :N].T)
    assert torch.equal(Bs, dg.shuffle_b(dev(B), dtype=dtype))


# tokens, d_model, d_ff; the tokens are the K of dW, so a multiple of 16 (bf16)
SMALL = [(304, 192, 320), (80, 270, 128), (1024, 256, 512)]


@pytest.mark.parametrize("T,D,F", SMALL, ids=lambda v: str(v))
def test_grad_input_small(T, D, F):
    """dX [T, D] = dY [T, F] W [F, D] for the up projection W [F, D]."""
    for smallint in (True, False):
        dist = "smallint" if smallint else "normal"
        dY, Wt = datagen.make_bf16_pair(T, D, F, dist, dist, config=T + D)   # Wt plays W^T [D, F]
        W = oracle.transpose(Wt)                                             # W [F, D]
        print(f"[grad_input T={T} D={D} F={F} smallint={smallint}]", flush=True)
        dX = dg.grad_input(dev_bf16(dY), dev_bf16(W))
        torch.cuda.synchronize()
        got = host_bits(dX)
        ref = oracle_full("bf16", dY, Wt)                                    # dY (W^T)^T = dY W
        if smallint:
            check_exact(got, ref, "dX")
        else:
            check_close("bf16", got, ref, oracle_full("bf16", abs_bits("bf16", dY),
                                                      abs_bits("bf16", Wt)), F, what="dX")


@pytest.mark.parametrize("T,D,F", SMALL, ids=lambda v: str(v))
def test_grad_weight_small(T, D, F):
    """dW [F, D] = dY^T [F, T] X [T, D]: the sum runs over the tokens."""
    for smallint in (True, False):
        dist = "smallint" if smallint else "normal"
        dY, X = datagen.make_bf16_pair(T, T, F, dist, dist, config=T + F)    # dY [T, F]
        X = datagen.make_bf16_pair(T, D, D, dist, dist, config=T + F + 1)[0]  # X [T, D]
        print(f"[grad_weight T={T} D={D} F={F} smallint={smallint}]", flush=True)
        dW = dg.grad_weight(dev_bf16(dY), dev_bf16(X))
        torch.cuda.synchronize()
        got = host_bits(dW)
        A, Bm = oracle.transpose(dY), oracle.transpose(X)                    # dY^T [F, T], X^T [D, T]
        ref = oracle_full("bf16", A, Bm)
        if smallint:
            check_exact(got, ref, "dW")
        else:
            check_close("bf16", got, ref, oracle_full("bf16", abs_bits("bf16", A),
                                                      abs_bits("bf16", Bm)), T, what="dW")


def test_grad_input_fp8_exact():
    """e4m3 dX through the primitives: shuffle_b_t of the e4m3 W, then the
    scaled GEMM (power-of-two scales, small integers: exact)."""
    T, D, F = 200, 160, 256
    dY, Wt, _, _ = datagen.make_e4m3_pair(T, D, F, config=41, smallint=True)
    W = oracle.transpose(Wt)
    Bs = dg.shuffle_b_t(dev_u8(W), dtype="fp8")
    sa = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    sb = torch.tensor([4.0], dtype=torch.float32, device="cuda")
    dX = dg.gemm_fp8_scaled(dev_u8(dY), Bs, D, sa, sb)
    torch.cuda.synchronize()
    check_exact(host_bits(dX), oracle_full("fp8", dY, Wt, 0.5, 4.0), "fp8 dX")


def _lines(n, tile=256):
    return sample_lines(n, tiles=(tile, 64), n_random=2)


def test_gpt3xl_grad_input_sampled():
    """dX [10240, 2048] = dY [10240, 8192] W [8192, 2048] (the TraceLens table's
    mm 10240 x 2048 x 8192)."""
    T, D, F = 10240, 2048, 8192
    dY, Wt = datagen.make_bf16_pair(T, D, F, "normal", "normal", config=71, sigma_b=0.02)
    W = oracle.transpose(Wt)
    print(f"[grad_input GPT-3-XL {T}x{D}x{F}]", flush=True)
    dX = dg.grad_input(dev_bf16(dY), dev_bf16(W))
    torch.cuda.synchronize()
    got = host_bits(dX)
    rows, cols = _lines(T), _lines(D)
    ms, ns, vals, absv = oracle_lines("bf16", dY, Wt, rows, cols)
    check_close("bf16", got[ms, ns][None, :], vals[None, :], absv[None, :], F, what="dX GPT-3-XL")


def test_gpt3xl_grad_weight_sampled():
    """dW [8192, 2048] = dY^T [8192, 10240] X [10240, 2048] (the table's mm
    8192 x 2048 x 10240)."""
    T, D, F = 10240, 2048, 8192
    dY = datagen.make_bf16_pair(T, 16, F, "normal", "normal", config=72)[0]   # [T, F]
    X = datagen.make_bf16_pair(T, 16, D, "normal", "normal", config=73)[0]    # [T, D]
    print(f"[grad_weight GPT-3-XL {F}x{D}x{T}]", flush=True)
    dW = dg.grad_weight(dev_bf16(dY), dev_bf16(X))
    torch.cuda.synchronize()
    got = host_bits(dW)
    A, Bm = oracle.transpose(dY), oracle.transpose(X)
    rows, cols = _lines(F), _lines(D)
    ms, ns, vals, absv = oracle_lines("bf16", A, Bm, rows, cols)
    check_close("bf16", got[ms, ns][None, :], vals[None, :], absv[None, :], T, what="dW GPT-3-XL")
