"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds none of the GEMM's arithmetic: it only draws numbers and casts
them to the input storage types, so that the oracle and the HIP path read
identical bytes.  The workloads it serves are the model-shaped GEMMs the pages
measure (LLaMA-2-7B MLP up/gate, GPT-2 lm_head and other ragged shapes); the
draws stand in for activations and trained weights.

Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser as published in Vigna's
splitmix64.c).  Output i of a stream with seed s is mix(s + (i + 1) * gamma)
with gamma = 0x9E3779B97F4A7C15.

Distributions:
  uniform [-1, 1):  u = (x >> 11) * 2^-53, value 2u - 1
  normal N(0, s^2): Box-Muller on consecutive pairs, both outputs used
  small integer:    ((x >> 32) mod 9) - 4, i.e. values in {-4..4}
Storage casts (torch CPU, both round to nearest even):
  bf16: fp64 -> fp32 -> bf16
  fp8:  per-tensor amax; q = e4m3(fp32(x) * (448 / amax)); dequant scale amax / 448
"""
from __future__ import annotations

import numpy as np
import torch

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
E4M3_MAX = 448.0


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n outputs of a splitmix64 stream started at ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _count(shape) -> int:
    return int(np.prod(shape, dtype=np.int64))


def uniform(seed: int, shape) -> np.ndarray:
    x = splitmix64(seed, _count(shape))
    u = (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return (2.0 * u - 1.0).reshape(shape)


def normal(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    n = _count(shape)
    x = splitmix64(seed, n + (n & 1))
    u = (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u1 = 1.0 - u[0::2]            # (0, 1]: keeps log finite
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(u.size, np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return (z[:n] * sigma).reshape(shape)


def small_int(seed: int, shape) -> np.ndarray:
    x = splitmix64(seed, _count(shape))
    return (((x >> np.uint64(32)) % np.uint64(9)).astype(np.int64) - 4).astype(np.float64).reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest even); returns the uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3(x: np.ndarray):
    """Per-tensor amax quantisation to OCP e4m3.

    Returns (codes uint8, dequant_scale float32): codes * scale approximates x.
    """
    xf = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    amax = float(xf.abs().max()) if xf.numel() else 1.0
    if amax == 0.0:
        amax = 1.0
    amax32 = np.float32(amax)
    inv = np.float32(E4M3_MAX) / amax32
    q = (xf * torch.tensor(inv, dtype=torch.float32)).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).numpy().copy()
    scale = np.float32(amax32 / np.float32(E4M3_MAX))
    return codes, float(scale)


def e4m3_exact(x: np.ndarray) -> np.ndarray:
    """Codes of values that are already exact e4m3 numbers (small integers)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ------------------------------------------------------- workload recipes
def seed_for(config: int, tensor: int) -> int:
    """Seed of tensor ``tensor`` (A = 1, B = 2) in workload ``config``."""
    return 1000 * config + tensor


def make_bf16_pair(M: int, N: int, K: int, dist_a: str, dist_b: str, config: int,
                   sigma_a: float = 1.0, sigma_b: float = 1.0):
    """bf16 bits of A [M, K] and the row-major weight B [N, K]."""
    def draw(dist, seed, shape, sigma):
        if dist == "uniform":
            return uniform(seed, shape)
        if dist == "normal":
            return normal(seed, shape, sigma)
        if dist == "smallint":
            return small_int(seed, shape)
        raise ValueError(dist)
    A = to_bf16_bits(draw(dist_a, seed_for(config, 1), (M, K), sigma_a))
    B = to_bf16_bits(draw(dist_b, seed_for(config, 2), (N, K), sigma_b))
    return A, B


def make_e4m3_pair(M: int, N: int, K: int, config: int, smallint: bool = False):
    """e4m3 codes of A [M, K], B [N, K] and their dequant scales.

    Normal inputs are N(0, 1) quantised per tensor to amax 448; the small-integer
    variant stores exact values in {-4..4} with scales 1.
    """
    if smallint:
        A = e4m3_exact(small_int(seed_for(config, 1), (M, K)))
        B = e4m3_exact(small_int(seed_for(config, 2), (N, K)))
        return A, B, 1.0, 1.0
    A, sa = to_e4m3(normal(seed_for(config, 1), (M, K)))
    B, sb = to_e4m3(normal(seed_for(config, 2), (N, K)))
    return A, B, sa, sb
