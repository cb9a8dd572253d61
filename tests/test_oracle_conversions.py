"""Pins for the oracle's dtype conversions and SiLU (CPU only).

The conversions are checked against independent library routines (torch's
bfloat16 cast, numpy's float16 cast, both round-to-nearest-even), over every
16-bit pattern for the widening direction, and on hand-made tie cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _all_bits():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_bf16_widen_all_patterns():
    bits = _all_bits()
    ours = oracle.to_f32(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_widen_all_patterns():
    bits = _all_bits()
    ours = oracle.to_f32(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    return np.concatenate([a, b, np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38,
                                           65504.0, 65519.99, 65520.0, 1e-8, 6e-8,
                                           2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26],
                                          np.float32)])


def test_bf16_round_matches_torch():
    x = _random_f32(200000, 1)
    ours = oracle.from_f32(x, oracle.BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN
    assert np.all(np.isnan(oracle.to_f32(ours[nan], oracle.BF16)))


def test_f16_round_matches_numpy():
    x = _random_f32(200000, 2)
    ours = oracle.from_f32(x, oracle.F16)
    ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.to_f32(ours[nan], oracle.F16)))


@pytest.mark.parametrize("value,expect", [
    (1.0 + 2.0 ** -8, 1.0),                   # exact tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),   # exact tie -> even (mantissa 2)
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),  # just above the tie
    (257.0, 256.0),                           # tie between 256 and 258
    (514.0, 512.0),                           # tie between 512 and 516
])
def test_bf16_tie_cases(value, expect):
    got = oracle.to_f32(oracle.from_f32(np.array([value, -value], np.float32), oracle.BF16),
                        oracle.BF16)
    assert got.tolist() == [expect, -expect]


@pytest.mark.parametrize("value,expect", [
    (2049.0, 2048.0), (2049.5, 2050.0), (4098.0, 4096.0), (65520.0, math.inf),
    (2.0 ** -25, 0.0), (3 * 2.0 ** -25, 2.0 ** -23),
])
def test_f16_tie_cases(value, expect):
    got = oracle.to_f32(oracle.from_f32(np.array([value], np.float32), oracle.F16), oracle.F16)
    assert got[0] == expect


def test_f32_storage_is_identity():
    x = _random_f32(1000, 3)
    assert np.array_equal(oracle.from_f32(x, oracle.F32).view(np.uint32), x.view(np.uint32))


def test_silu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 200.0, -200.0, 20.0], np.float32)
    u = np.ones_like(g)
    s = oracle.silu_mul(g, u)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-7            # 1 / (1 + e^-1)
    assert abs(s[2] - (-0.2689414213699951)) < 1e-7         # -1 / (1 + e)
    assert s[3] == 200.0                                     # e^-200 underflows
    assert s[4] == 0.0                                       # -200 / inf
    assert abs(s[5] - 20.0 / (1.0 + math.exp(-20.0))) < 2e-6


def test_silu_matches_definition():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(10000) * 6).astype(np.float32)
    u = rng.standard_normal(10000).astype(np.float32)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64))) * u
    got = oracle.silu_mul(g, u)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-30)) < 1e-6
