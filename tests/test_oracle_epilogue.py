"""Pins of the oracle's fused epilogue (oracle.c: orc_activation, orc_epilogue).

- Hand-worked cases (tests/golden/epilogue_small.json): the order scale,
  bias, activation, multiplier on a 2 x 2 product.
- Textbook activation values (logistic(1), the normal CDF at 1 and 2).
- Library routines: SiLU = x * scipy.special.expit(x); the erf GELU = x *
  scipy.stats.norm.cdf(x); the tanh GELU = torch's float64
  gelu(approximate="tanh"), with a planted coefficient slip shown to fail.
- Identities: f(x) - f(-x) = x for SiLU and both GELU forms (logistic(x) +
  logistic(-x) = 1, Phi(x) + Phi(-x) = 1, tanh odd), which catches a sign or
  argument slip; the tanh form stays within 1e-3 of the erf form but is not
  the same function.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "epilogue_small.json")


def bf16(x):
    return oracle.bf16_from_f64(np.asarray(x, np.float64))


def test_golden_cases():
    g = json.load(open(GOLD))
    A = bf16(g["A"])
    B = bf16(g["B"])
    C = oracle.gemm_bf16(A, B)
    assert np.array_equal(C, [[17.0, 23.0], [39.0, 53.0]])
    for case in g["cases"]:
        out = oracle.epilogue(
            C,
            scale_m=None if "scale_m" not in case else np.array(case["scale_m"], np.float32),
            scale_n=None if "scale_n" not in case else np.array(case["scale_n"], np.float32),
            bias=None if "bias" not in case else bf16(case["bias"]),
            act=case["act"],
            mul=None if "mul" not in case else bf16(case["mul"]))
        assert np.array_equal(out, np.array(case["out"])), case["name"]


def test_textbook_activation_values():
    acts = json.load(open(GOLD))["activations"]
    for x, y in acts["silu"]:
        assert oracle.activation(oracle.ACT_SILU, x) == pytest.approx(y, abs=1e-15)
    for x, y in acts["gelu_erf"]:
        assert oracle.activation(oracle.ACT_GELU_ERF, x) == pytest.approx(y, abs=1e-15)


def test_against_library_routines():
    x = np.linspace(-12, 12, 4001)
    np.testing.assert_allclose(oracle.activation(oracle.ACT_SILU, x), x * special.expit(x),
                               rtol=1e-14, atol=1e-300)
    # 1 + erf(x / sqrt 2) cancels for large negative x: the definition as
    # written loses up to |x| * 2^-52 absolutely there (norm.cdf does not)
    g = oracle.activation(oracle.ACT_GELU_ERF, x)
    ref = x * stats.norm.cdf(x)
    assert np.all(np.abs(g - ref) <= 1e-13 * np.abs(ref) + np.abs(x) * 2.0 ** -52)
    np.testing.assert_array_equal(oracle.activation(oracle.ACT_RELU, x), np.maximum(x, 0.0))
    np.testing.assert_array_equal(oracle.activation(oracle.ACT_NONE, x), x)


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_GELU_ERF, oracle.ACT_GELU_TANH])
def test_odd_part_identity(act):
    x = np.linspace(-8, 8, 1601)
    d = oracle.activation(act, x) - oracle.activation(act, -x)
    np.testing.assert_allclose(d, x, rtol=0, atol=1e-13)


def test_tanh_form_close_to_erf_form_but_distinct():
    x = np.linspace(-10, 10, 20001)
    t = oracle.activation(oracle.ACT_GELU_TANH, x)
    e = oracle.activation(oracle.ACT_GELU_ERF, x)
    diff = np.abs(t - e)
    assert diff.max() < 1e-3
    assert diff.max() > 1e-5
    assert oracle.activation(oracle.ACT_GELU_TANH, 0.0) == 0.0
    assert oracle.activation(oracle.ACT_GELU_TANH, 30.0) == pytest.approx(30.0, rel=1e-15)


def test_parts_compose_and_identity():
    rng = np.random.default_rng(5)
    C = rng.normal(size=(7, 9))
    assert np.array_equal(oracle.epilogue(C), C)
    sm = rng.uniform(0.5, 2, 7).astype(np.float32)
    sn = rng.uniform(0.5, 2, 9).astype(np.float32)
    bias = bf16(rng.normal(size=9))
    mul = bf16(rng.normal(size=(7, 12)))
    got = oracle.epilogue(C, sm, sn, bias, oracle.ACT_SILU, mul)
    pre = C * sm[:, None].astype(np.float64) * sn[None, :] + oracle.bf16_to_f64(bias)[None, :]
    want = pre * special.expit(pre) * oracle.bf16_to_f64(mul)[:, :9]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)
    ones = bf16(np.ones((7, 9)))
    assert np.array_equal(oracle.epilogue(C, mul=ones), C)


def test_gelu_tanh_against_torch():
    """The tanh form against torch's own float64 gelu(approximate="tanh"), an
    implementation written apart from this oracle: a slip in the cubic
    coefficient (0.0447 for 0.044715 moves the output by up to 4.7e-4) or in
    sqrt(2/pi) fails by orders of magnitude.  For large negative x both sides
    compute 1 + tanh(.) by cancellation, so the absolute slack there is one
    rounding of |x|."""
    import torch
    x = np.linspace(-12, 12, 48001)
    got = oracle.activation(oracle.ACT_GELU_TANH, x)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.all(np.abs(got - ref) <= 1e-14 * np.abs(ref) + np.abs(x) * 2.0 ** -52)
    pos = x > 0.5
    np.testing.assert_allclose(got[pos], ref[pos], rtol=1e-14, atol=0)


def test_gelu_tanh_planted_coefficient_slip_is_caught():
    """The check above rejects the plausible slip: the same formula with the
    cubic coefficient rounded to 0.0447 (computed here, not in the oracle)."""
    import torch
    x = np.linspace(-12, 12, 48001)
    slipped = 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.0447 * x ** 3)))
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert not np.all(np.abs(slipped - ref) <= 1e-14 * np.abs(ref) + np.abs(x) * 2.0 ** -52)
