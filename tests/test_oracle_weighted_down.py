"""Pins for the oracle's forward with the routing weight in the down epilogue
(CPU only): expert_out row = R(w * (h . Wd)), then an unweighted fp32 sum in
k order.

  * all-ones weights: the same bits as the weighted-combine forward (h, every
    expert_out row and y), since R(1 * o) = R(o) and fma(1, a, b) = a + b;
  * power-of-two weights: scaling by 2^-n commutes with rounding (no
    subnormals or overflow at these magnitudes), so every weighted row is
    exactly w times the unweighted one and y matches the weighted-combine
    forward bit for bit;
  * general weights: against a float64 evaluation of the same steps on the
    oracle's own h, with the 16-bit roundings done by torch; and within the
    16-bit bar of the dense float64 brute force;
  * masked slots: zero rows, never accumulated.
"""
import numpy as np
import torch

import oracle
from test_oracle_forward import _case, _rel, dense_brute_force


def _bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _both(x, wg, wu, wd, ids, w, dt=oracle.BF16):
    args = [_bits(a) for a in (x, wg, wu, wd)] if dt == oracle.BF16 else [x, wg, wu, wd]
    base = oracle.moe_forward(dt, *args, ids, w, want_pairs=True)
    wdn = oracle.moe_forward(dt, *args, ids, w, want_pairs=True, weighted_down=True)
    return base, wdn


def test_unit_weights_equal_weighted_combine():
    x, wg, wu, wd, ids, _ = _case(12, 64, 32, 4, 2, seed=1, mask=0.2)
    w = np.ones(ids.shape, np.float32)
    (y0, h0, e0), (y1, h1, e1) = _both(x, wg, wu, wd, ids, w)
    assert np.array_equal(h0, h1) and np.array_equal(e0, e1) and np.array_equal(y0, y1)


def test_power_of_two_weights_exact():
    x, wg, wu, wd, ids, _ = _case(10, 64, 48, 5, 3, seed=2, mask=0.1)
    rng = np.random.default_rng(3)
    w = (2.0 ** -rng.integers(0, 5, size=ids.shape)).astype(np.float32)
    (y0, h0, e0), (y1, h1, e1) = _both(x, wg, wu, wd, ids, w)
    assert np.array_equal(h0, h1)
    assert np.array_equal(e1, e0 * np.repeat(w.reshape(-1, 1), e0.shape[1], axis=1))
    assert np.array_equal(y0, y1)


def test_general_weights_against_float64_steps():
    T, H, D, E, K = 9, 64, 32, 4, 3
    x, wg, wu, wd, ids, w = _case(T, H, D, E, K, seed=4, mask=0.15)
    (y0, _, _), (y1, h1, e1) = _both(x, wg, wu, wd, ids, w)
    ref = np.zeros((T, H), np.float64)
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            if e < 0:
                assert np.all(e1[t * K + k] == 0) and np.all(h1[t * K + k] == 0)
                continue
            o = wd[e].astype(np.float64) @ h1[t * K + k].astype(np.float64)
            row = _bf16(np.float32(w[t, k]) * o.astype(np.float32))
            # the dot product in fp32 differs from float64 by rounding only:
            # at most one bf16 ulp of the row
            assert np.all(np.abs(e1[t * K + k] - row) <= 2.0 ** -7 * np.abs(row) + 1e-30)
            ref[t] += e1[t * K + k].astype(np.float64)
    # the combine: fp32 sums in k order of the stored rows, vs float64
    assert np.abs(y1 - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
    # both forms stay within the 16-bit bar of the exact forward
    exact = dense_brute_force(x, wg, wu, wd, ids, w)
    assert _rel(y1, exact) <= 5e-3 and _rel(y0, exact) <= 5e-3
    assert not np.array_equal(y0, y1)        # the two forms round at different points


def test_fp32_storage_matches_brute_force():
    x, wg, wu, wd, ids, w = _case(8, 32, 16, 3, 2, seed=5, mask=0.2)
    (y0, _, _), (y1, _, _) = _both(x, wg, wu, wd, ids, w, dt=oracle.F32)
    exact = dense_brute_force(x, wg, wu, wd, ids, w)
    assert _rel(y1, exact) <= 1e-5 and _rel(y0, exact) <= 1e-5


def test_all_masked_token_is_zero():
    x, wg, wu, wd, ids, w = _case(4, 32, 16, 3, 2, seed=6)
    ids[2] = -1
    (_, _, _), (y1, _, e1) = _both(x, wg, wu, wd, ids, w)
    assert np.all(y1[2] == 0) and np.all(e1[4:6] == 0)
