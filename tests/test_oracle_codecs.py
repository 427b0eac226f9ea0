"""Pins for the oracle's number codecs (CPU only).

bf16: exhaustive round trip over all 65536 patterns, hand-worked ties (round to
nearest even, the reading of the epilogue's "truncate to the output type" in the
"GEMM Optimization Guide" page, section 7.1), and a bit-for-bit match with
torch's float32 -> bfloat16 conversion on a million values.
e4m3 (OCP E4M3FN): the 256-code table against the format's definition and
against torch's float8_e4m3fn decoding, hand-worked ties and saturation.
"""
import numpy as np
import torch

import oracle


def test_bf16_exhaustive_round_trip():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(codes)
    tvals = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(vals)
    np.testing.assert_array_equal(np.isnan(tvals), nan)
    np.testing.assert_array_equal(vals[~nan], tvals[~nan])
    back = oracle.bf16_from_f64(vals[~nan])
    np.testing.assert_array_equal(back, codes[~nan])
    assert nan.sum() == 2 * 127          # exponent all ones, mantissa != 0
    assert (oracle.bf16_from_f64(vals[nan]) & 0x7FFF == 0x7FC0).all()


def _f32(bits):
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def test_bf16_ties_to_even():
    cases = {
        0x3F808000: 0x3F80,   # 1 + 2^-8 exactly half way: keep even 0x3F80
        0x3F818000: 0x3F82,   # half way above odd 0x3F81: round up to even
        0x3F808001: 0x3F81,   # just above half: up
        0xBF808000: 0xBF80,   # sign symmetric
        0x00008000: 0x0000,   # subnormal tie to even (zero)
        0x00018000: 0x0002,   # subnormal tie up to even
        0x7F7F8000: 0x7F80,   # max finite + half ulp overflows to inf
        0x7F7F7FFF: 0x7F7F,
    }
    for f32bits, bf in cases.items():
        assert oracle._load().orc_bf16_from_f64(_f32(f32bits)) == bf, hex(f32bits)
    # integers above 256 are not all representable: 257 -> 256, 259 -> 260
    assert oracle.bf16_to_f64(oracle.bf16_from_f64(np.array([257.0, 259.0, 261.0, 263.0]))).tolist() \
        == [256.0, 260.0, 260.0, 264.0]


def test_bf16_matches_torch_on_random_floats():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.bf16_from_f64(f.astype(np.float64))
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def _e4m3_definition(c):
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    table = np.array([_e4m3_definition(int(c)) for c in codes])
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(table))
    ok = ~np.isnan(table)
    np.testing.assert_array_equal(vals[ok], table[ok])
    tvals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals[ok], tvals[ok])
    assert vals[0x7E] == 448.0 and vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.nanmax(vals) == 448.0
    back = oracle.e4m3_from_f64(vals[ok])
    zero_neg = codes[ok] == 0x80          # -0 encodes back to 0x80
    np.testing.assert_array_equal(back[~zero_neg], codes[ok][~zero_neg])


def test_e4m3_ties_and_saturation():
    enc = oracle._load().orc_e4m3_from_f64
    assert enc(1.0625) == 0x38          # half way 1.0 / 1.125: even mantissa 0 wins
    assert enc(1.1875) == 0x3A          # half way 1.125 / 1.25: even (1.25) wins
    assert enc(500.0) == 0x7E           # saturate to 448
    assert enc(-1e9) == 0xFE
    assert enc(2.0 ** -10) == 0x00      # half of the smallest subnormal: tie to even zero
    assert enc(3 * 2.0 ** -10) == 0x02  # 1.5 quanta -> 2 quanta
    assert enc(float("nan")) == 0x7F


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 100, 200_000), rng.normal(0, 0.01, 200_000)])
    x = np.clip(x, -447.0, 447.0).astype(np.float32)
    ours = oracle.e4m3_from_f64(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)
