"""Pins for the oracle's FP8 E4M3 storage type (OCP 8-bit floating point
specification, format E4M3: bias 7, 3 fraction bits, no infinities, one NaN
pattern per sign, largest finite 448), used by the scaled / FP8 variants of
moe_reduce_fused (TileOPs-Metax PR #55, section 1).

  * decode: every one of the 256 codes against torch.float8_e4m3fn's decode,
    and closed-form values (1, 448, the smallest normal and subnormal);
  * encode: round trip of every finite code, exact midpoints between
    neighbouring codes going to the even code, random in-range values
    against torch's cast, saturation of out-of-range values and infinities to
    +-448, NaN to the NaN pattern.
"""
import math

import numpy as np
import torch

import oracle


def _decode(codes):
    return oracle.to_f32(np.asarray(codes, np.uint8), oracle.FP8)


def _encode(x):
    return oracle.from_f32(np.asarray(x, np.float32), oracle.FP8)


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = _decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2          # 0x7f, 0xff
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_decode_closed_forms():
    v = _decode([0x38, 0x7e, 0x08, 0x01, 0x07, 0x00, 0x80, 0xbe, 0x40])
    assert v.tolist() == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 0.0, -0.0, -1.75, 2.0]
    assert math.copysign(1.0, float(v[6])) == -1.0


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7f != 0x7f], np.uint8)
    assert np.array_equal(_encode(_decode(codes)), codes)


def test_encode_midpoints_round_to_even():
    # Positive finite codes in increasing value order are 0x00..0x7e.
    vals = _decode(np.arange(0x7f, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)   # exact in fp32
    got = _encode(mids)
    lo = np.arange(0x7e, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(_encode(-mids), want | 0x80)


def test_encode_random_in_range_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(_encode(x), ref)


def test_encode_saturates_and_keeps_nan():
    got = _encode([448.0, 449.0, 464.0, 500.0, 1e30, np.inf, -np.inf, -1e9, np.nan, -np.nan])
    assert got.tolist() == [0x7e, 0x7e, 0x7e, 0x7e, 0x7e, 0x7e, 0xfe, 0xfe, 0x7f, 0xff]
    # below the smallest subnormal's half: zero, sign kept
    assert _encode([2.0 ** -11, -2.0 ** -11]).tolist() == [0x00, 0x80]
