"""Helpers for the GPU parity tests: move synthetic inputs to the device, run
the HIP path through the C ABI, and compare with the oracle.

Comparison rules (fixed here, used by every GPU test):
  * small-integer inputs: the exact sum is an integer below 2^24 in magnitude,
    so every fp32 accumulation order gives it exactly and the bf16 output has
    one correct value: bits must equal the oracle's round-to-nearest-even of
    the fp64 sum (-0 and +0 identified);
  * full-size workloads are compared on every element too (the oracle's
    whole product on the host's threads), with the accumulation term of the
    element bound taken from row norms (check_close_full);
  * general inputs: relative Frobenius error over the real M x N region
    against the unrounded fp64 oracle, at most 2e-3 (bf16) or 3e-2 (e4m3,
    after scales); and element by element
        |C - Cref| <= 2^-8 |Cref| + g * sum_k |a_k b_k| * scale
    i.e. one bf16 rounding (half an ulp is at most 2^-8 of the value) plus
    an accumulation term, so a wrong column or row cannot hide inside an
    aggregate.  bf16: g = (K + 2) * 2^-24, the worst-case fp32 accumulation
    error in any order.  e4m3: the gfx950 f8f6f4 MFMA forms the sum of the
    128 products of one instruction with a narrower adder than fp32 (measured
    on MI355X: 448^2 + 4 - 448^2 gives 0 when the three products fall in one
    half of the instruction's K, while fp32 would keep the 4), and only the
    accumulation across instructions is fp32; so g = 2^-12 + (K/128 + 2) *
    2^-24.  Any indexing mistake is off by a sizeable fraction of
    sum |a_k b_k|, far above either g.
"""
from __future__ import annotations

import numpy as np
import torch

import dense_gemm_linear_amd as dg
import oracle

SENTINEL = 0xFFFF     # a NaN bit pattern the kernels never write
REL_FRO = {"bf16": 2e-3, "fp8": 3e-2}


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def alloc_c(M: int, N: int, ldc: int | None = None, guard: int = 16, col0: int = 0):
    """C as a view into a sentinel-filled buffer of (M + guard) x ldc_alloc."""
    ldc = N + col0 if ldc is None else ldc
    assert ldc >= N + col0
    buf = torch.full(((M + guard), ldc), SENTINEL - 65536, dtype=torch.int16, device="cuda")
    view = buf.view(torch.bfloat16)[:M, col0:col0 + N]
    return buf, view


def guard_untouched(buf: torch.Tensor, M: int, N: int, col0: int = 0) -> bool:
    h = buf.cpu().numpy().view(np.uint16).copy()
    h[:M, col0:col0 + N] = SENTINEL
    return bool((h == SENTINEL).all())


def run(dt: str, A: np.ndarray, B: np.ndarray, tile=None, sa: float = 1.0, sb: float = 1.0,
        ldc: int | None = None, col0: int = 0, guard: int = 16, workspace=None):
    """Shuffle B on the device, run the GEMM, return (C bits [M, N], guard ok).
    workspace: a uint8 device tensor for split-K tiles (None: the binding
    allocates one when a forced split-K tile needs it)."""
    M, K = A.shape
    N = B.shape[0]
    if dt == "bf16":
        Ad, Bd = dev_bf16(A), dev_bf16(B)
    else:
        Ad, Bd = dev_u8(A), dev_u8(B)
    Bs = dg.shuffle_b(Bd, dtype=dt)
    buf, C = alloc_c(M, N, ldc, guard, col0)
    if dt == "bf16":
        dg.gemm_bf16(Ad, Bs, N, out=C, tile=tile, workspace=workspace)
    else:
        s_a = torch.tensor([sa], dtype=torch.float32, device="cuda")
        s_b = torch.tensor([sb], dtype=torch.float32, device="cuda")
        dg.gemm_fp8_scaled(Ad, Bs, N, s_a, s_b, out=C, tile=tile, workspace=workspace)
    torch.cuda.synchronize()
    return host_bits(C), guard_untouched(buf, M, N, col0)


def oracle_full(dt: str, A, B, sa: float = 1.0, sb: float = 1.0):
    if dt == "bf16":
        return oracle.gemm_bf16(A, B)
    return oracle.gemm_e4m3(A, B, sa, sb)


def abs_bits(dt: str, X: np.ndarray) -> np.ndarray:
    """Same storage format with the sign bit cleared (|x|)."""
    return X & (0x7FFF if dt == "bf16" else 0x7F)


def check_exact(Cbits: np.ndarray, Cref: np.ndarray, what: str = ""):
    want = oracle.bf16_from_f64(Cref)
    got = Cbits.copy()
    got[got == 0x8000] = 0
    want[want == 0x8000] = 0
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}"


def check_close(dt: str, Cbits: np.ndarray, Cref: np.ndarray, absref: np.ndarray, K: int,
                scale: float = 1.0, what: str = ""):
    got = oracle.bf16_to_f64(Cbits)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = got - Cref
    fro = np.linalg.norm(err) / max(np.linalg.norm(Cref), 1e-300)
    assert fro <= REL_FRO[dt], f"{what}: relative Frobenius error {fro:.3e}"
    g = (K + 2) * 2.0 ** -24 if dt == "bf16" else 2.0 ** -12 + (K / 128 + 2) * 2.0 ** -24
    bound = 2.0 ** -8 * np.abs(Cref) + g * absref * scale + 1e-30
    viol = np.argwhere(np.abs(err) > bound)
    assert viol.size == 0, f"{what}: {len(viol)} elements out of bound, first {viol[:5].tolist()}"
    return fro


def row_norms(dt: str, X: np.ndarray) -> np.ndarray:
    """Euclidean norm of every row of a bf16-bit or e4m3-code array."""
    v = oracle.bf16_to_f64(X) if dt == "bf16" else oracle.e4m3_to_f64(X)
    return np.sqrt(np.einsum("ij,ij->i", v, v))


def check_close_full(dt: str, Cbits: np.ndarray, Cref: np.ndarray, A, B, K: int,
                     scale: float = 1.0, what: str = ""):
    """check_close over every element of a full-size product, with
    sum_k |a_k b_k| replaced by its Cauchy-Schwarz bound |a_m| |b_n| (row
    norms): an upper bound of the element bound that needs no second
    full product of absolute values.  For the workloads' random inputs it is
    about 1.6 times the exact sum, and the accumulation term stays far below
    any indexing mistake (which is off by a fraction of the whole sum)."""
    absref = np.multiply.outer(row_norms(dt, A), row_norms(dt, B))
    return check_close(dt, Cbits, Cref, absref, K, scale, what)


def sample_lines(extent: int, tiles=(256, 128, 64, 32, 16), n_random: int = 6, seed: int = 0):
    """Indices on both sides of tile boundaries near the start, middle and end
    of the extent for every tile size, the two ends, and a few random ones."""
    s = {0, extent - 1}
    for t in tiles:
        bounds = list(range(t, extent, t))
        picks = bounds[:2] + bounds[len(bounds) // 2:len(bounds) // 2 + 1] + bounds[-2:]
        for b in picks:
            s.update({b - 1, b})
    rng = np.random.default_rng(seed + extent)
    s.update(rng.integers(0, extent, size=n_random).tolist())
    return np.array(sorted(i for i in s if 0 <= i < extent), np.int64)


def oracle_lines(dt: str, A, B, rows, cols, scale: float = 1.0):
    """Oracle values on whole rows `rows` and whole columns `cols`, and the
    unscaled sums of |a_k b_k| there (for the element bound)."""
    M, N = A.shape[0], B.shape[0]
    ms = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols))])
    ns = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M)])
    code = oracle.ORC_BF16 if dt == "bf16" else oracle.ORC_E4M3
    vals = oracle.gemm_points(code, A, B, ms, ns, scale)
    absv = oracle.gemm_points(code, abs_bits(dt, A), abs_bits(dt, B), ms, ns, 1.0)
    return ms, ns, vals, absv
