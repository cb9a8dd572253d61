"""Pins for the oracle's FP8 expert weights (CPU only): the per-row quantizer
and the forward over FP8 codes with per-row scales.

  * quantizer: the row maximum maps to the largest code (448), every code
    decodes within half an E4M3 step of w / s (checked against numpy's own
    rounding of the exact quotient), zero rows give code 0 and scale 1,
    values that are exactly E4M3 multiples of the scale reconstruct exactly;
  * forward: with power-of-two scales and weights that are exactly
    scale x E4M3 value, the FP8 forward equals the forward over the same
    weights stored in bf16 bit for bit (scaling by a power of two commutes
    with rounding), so a misplaced or missing scale fails; against a float64
    brute force over the decoded weights within the graded tolerance.
"""
import numpy as np
import torch

import oracle

E4M3_MAX = 448.0


def _e4m3_grid():
    """All finite non-negative E4M3 values, from the format definition."""
    vals = [m * 2.0 ** -9 for m in range(8)]                       # subnormals
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                           # NaN
            vals.append((1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(sorted(set(vals)))


GRID = _e4m3_grid()


def _decode(codes):
    return oracle.to_f32(codes, oracle.FP8)


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3_grid_matches_decoder():
    codes = np.arange(256, dtype=np.uint8)
    dec = _decode(codes)
    finite = ~np.isnan(dec)
    assert finite.sum() == 254
    assert np.array_equal(np.unique(np.abs(dec[finite])), GRID)
    assert GRID.max() == E4M3_MAX


def test_quantizer_scales_and_codes():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((6, 96)) * rng.uniform(0.01, 3, size=(6, 1))).astype(np.float32)
    w[3] = 0.0
    q, s = oracle.quantize_fp8_rows(oracle.F32, w)
    amax = np.abs(w).max(axis=1)
    assert np.array_equal(s[[0, 1, 2, 4, 5]], (amax / np.float32(448.0)).astype(np.float32)[[0, 1, 2, 4, 5]])
    assert s[3] == 1.0 and np.all(q[3] == 0)
    dec = _decode(q)
    for r in (0, 1, 2, 4, 5):
        ratio = w[r].astype(np.float32) / s[r]                     # fp32 quotient, as specified
        assert np.abs(dec[r]).max() == E4M3_MAX                    # the row maximum takes 448
        # each code is the nearest E4M3 value of the quotient (ties to even code)
        idx = np.searchsorted(GRID, np.abs(ratio).astype(np.float64))
        lo = GRID[np.clip(idx - 1, 0, len(GRID) - 1)]
        hi = GRID[np.clip(idx, 0, len(GRID) - 1)]
        best = np.minimum(np.abs(np.abs(ratio) - lo), np.abs(np.abs(ratio) - hi))
        assert np.all(np.abs(np.abs(dec[r]) - np.abs(ratio)) <= best + 1e-12)
        assert np.all(np.sign(dec[r]) * np.sign(ratio) >= 0)


def test_quantizer_exact_on_representable_rows():
    rng = np.random.default_rng(1)
    s_true = np.float32(2.0 ** -5)
    v = rng.choice(np.concatenate([-GRID, GRID]), size=(4, 64))
    v[:, 0] = E4M3_MAX                                             # pins the row maximum
    w = (v * s_true).astype(np.float32)
    q, s = oracle.quantize_fp8_rows(oracle.BF16, _bf16_bits(w))
    assert np.all(s == s_true)
    assert np.array_equal(_decode(q), v.astype(np.float32))


def _pow2_fp8_weights(rng, shape):
    """Weights = 2^-k x E4M3 value with k per row: exactly representable in
    bf16 and reconstructed exactly by the quantizer."""
    v = rng.choice(np.concatenate([-GRID[:80], GRID[:80]]), size=shape)   # <= 2^-0 range
    v[..., 0] = E4M3_MAX
    k = rng.integers(6, 12, size=shape[:-1])
    return (v * 2.0 ** (-k[..., None])).astype(np.float32)


def test_forward_w8_equals_bf16_forward_on_exact_weights():
    rng = np.random.default_rng(2)
    T, H, D, E, K = 10, 64, 32, 3, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = _pow2_fp8_weights(rng, (E, D, H))
    wu = _pow2_fp8_weights(rng, (E, D, H))
    wd = _pow2_fp8_weights(rng, (E, H, D))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[2, 1] = -1
    w = rng.uniform(0.1, 1, size=(T, K)).astype(np.float32)
    bits = [_bf16_bits(a) for a in (x, wg, wu, wd)]
    q = [oracle.quantize_fp8_rows(oracle.BF16, b) for b in bits[1:]]
    for (codes, scales), ref in zip(q, (wg, wu, wd)):
        assert np.array_equal(_decode(codes) * scales[..., None], ref)
    y16, h16, e16 = oracle.moe_forward(oracle.BF16, *bits, ids, w, want_pairs=True)
    y8, h8, e8 = oracle.moe_forward_w8(oracle.BF16, bits[0], q[0][0], q[1][0], q[2][0], q[0][1],
                                       q[1][1], q[2][1], ids, w, want_pairs=True)
    assert np.array_equal(h8, h16) and np.array_equal(e8, e16) and np.array_equal(y8, y16)


def test_forward_w8_against_float64_brute_force():
    rng = np.random.default_rng(3)
    T, H, D, E, K = 12, 128, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = _bf16_bits(x)
    xf = oracle.to_f32(xb, oracle.BF16).astype(np.float64)
    ws = [(rng.standard_normal(sh) / np.sqrt(sh[-1])).astype(np.float32)
          for sh in ((E, D, H), (E, D, H), (E, H, D))]
    q = [oracle.quantize_fp8_rows(oracle.F32, a) for a in ws]
    deq = [_decode(c).astype(np.float64) * s[..., None].astype(np.float64) for c, s in q]
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1, size=(T, K)).astype(np.float32)
    y8 = oracle.moe_forward_w8(oracle.BF16, xb, q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                               q[2][1], ids, w)
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            g = deq[0][e] @ xf[t]
            u = deq[1][e] @ xf[t]
            h = g / (1 + np.exp(-g)) * u
            ref[t] += w[t, k] * (deq[2][e] @ h)
    diff = y8 - ref
    assert np.abs(diff).max() <= 2e-2
    assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 5e-3
