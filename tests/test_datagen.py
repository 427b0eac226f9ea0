"""Pins for the seeded input generators (CPU): published splitmix64 outputs,
moments within three standard errors, value sets, determinism, and the fp8
quantiser agreeing with the oracle's own e4m3 encoder."""
import json
import os

import numpy as np

import datagen
import oracle


def test_splitmix64_published_outputs(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "splitmix64.json")))
    got = [int(v) for v in datagen.splitmix64(g["seed"], len(g["outputs_hex"]))]
    assert got == [int(h, 16) for h in g["outputs_hex"]]


def test_determinism():
    a = datagen.make_bf16_pair(7, 9, 32, "normal", "uniform", config=3)
    b = datagen.make_bf16_pair(7, 9, 32, "normal", "uniform", config=3)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = datagen.make_bf16_pair(7, 9, 32, "normal", "uniform", config=4)
    assert not np.array_equal(a[0], c[0])


def test_moments():
    n = 400_000
    x = datagen.normal(5, (n,), 0.02)
    se = 0.02 / np.sqrt(n)
    assert abs(x.mean()) < 3 * se
    assert abs(x.std() - 0.02) < 3 * 0.02 / np.sqrt(2 * n) + 1e-5
    u = datagen.uniform(6, (n,))
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 3 * np.sqrt(1 / 3) / np.sqrt(n)
    s = datagen.small_int(7, (n,))
    assert set(np.unique(s).tolist()) == set(range(-4, 5))
    assert abs(s.mean()) < 3 * np.sqrt(20 / 3) / np.sqrt(n)


def test_bf16_storage_cast_is_rne_of_fp32():
    x = datagen.normal(8, (10000,))
    bits = datagen.to_bf16_bits(x)
    np.testing.assert_array_equal(bits, oracle.bf16_from_f64(x.astype(np.float32).astype(np.float64)))


def test_e4m3_quantiser_against_oracle_encoder():
    x = datagen.normal(9, (300, 200))
    codes, scale = datagen.to_e4m3(x)
    amax = np.float32(np.abs(x.astype(np.float32)).max())
    inv = np.float32(448.0) / amax
    scaled = (x.astype(np.float32) * inv).astype(np.float64)
    np.testing.assert_array_equal(codes, oracle.e4m3_from_f64(scaled))
    assert codes.view(np.uint8).max() in (0x7E, 0xFE)
    assert (codes & 0x7F).max() == 0x7E                    # amax lands on 448
    assert abs(scale - float(amax) / 448.0) <= 1e-7 * scale
    ai, bi, sa, sb = datagen.make_e4m3_pair(4, 5, 64, config=5, smallint=True)
    assert sa == sb == 1.0
    assert set(np.unique(oracle.e4m3_to_f64(ai)).tolist()) <= set(range(-4, 5))
