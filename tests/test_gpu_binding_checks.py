"""Binding-level operand checks that need device tensors: each mistake below
raises ValueError in the binding, before any launch (the C ABI sees only
pointers and could not tell).  Nothing here reaches a kernel."""
import pytest
import torch

import dense_gemm_linear_amd as dg

pytestmark = pytest.mark.gpu


def test_bs_must_be_a_large_enough_device_buffer():
    A = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    need = dg.shuffle_b_bytes(64, 128)
    with pytest.raises(ValueError, match="needs"):
        dg.gemm_bf16(A, torch.zeros(need - 16, dtype=torch.uint8, device="cuda"), 64)
    with pytest.raises(ValueError, match="device"):
        dg.gemm_bf16(A, torch.zeros(need, dtype=torch.uint8), 64)          # host Bs
    with pytest.raises(ValueError, match="contiguous"):
        dg.gemm_bf16(A, torch.zeros(2 * need, dtype=torch.uint8, device="cuda")[::2], 64)
    # a Bs shuffled for a smaller K is too small for this A
    with pytest.raises(ValueError, match="needs"):
        dg.gemm_bf16(A, torch.zeros(dg.shuffle_b_bytes(64, 64), dtype=torch.uint8,
                                    device="cuda"), 64)
    torch.cuda.synchronize()


def test_scales_must_be_float32_device_tensors():
    A = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    Bs = torch.zeros(dg.shuffle_b_bytes(64, 128, "fp8"), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="scale_a"):
        dg.gemm_fp8_scaled(A, Bs, 64, torch.ones(1, dtype=torch.float32), one)   # host scale
    with pytest.raises(ValueError, match="scale_b"):
        dg.gemm_fp8_scaled(A, Bs, 64, one, torch.ones(1, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="element type"):
        dg.gemm_fp8_scaled(A.view(torch.int16)[:, :32].contiguous(), Bs, 64, one, one)
    # the well-formed call still runs
    C = dg.gemm_fp8_scaled(A, Bs, 64, one, one)
    torch.cuda.synchronize()
    assert C.shape == (8, 64) and int(C.view(torch.int16).abs().max()) == 0
