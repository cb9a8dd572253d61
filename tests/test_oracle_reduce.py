"""Pins for the oracle's moe_reduce_fused (CPU only).

  * exact results on integer-valued rows with power-of-two weights (every
    partial sum is exact in fp32, so the answer is known exactly);
  * the gather-then-sum formulation (the vectorised reference the
    TileOPs-Metax moe_reduce_fused PR compares against) in float64;
  * masked slots never read (a NaN row at the index a wrapped -1 would hit),
    NULL weights equal all-ones, K = 1, out-of-range positions rejected;
  * the PR's correctness shapes (T x K x H).
"""
import numpy as np
import pytest
import torch

import oracle


def gather_sum(X, pos, w):
    X = np.asarray(X, np.float64)
    T, K = pos.shape
    g = X[np.clip(pos, 0, None)]                       # [T, K, H]
    wk = (np.ones((T, K)) if w is None else w.astype(np.float64)) * (pos >= 0)
    return np.einsum("tk,tkh->th", wk, g)


def _bits(a, tdt):
    return torch.from_numpy(np.asarray(a, np.float32)).to(tdt).view(torch.int16).numpy().view(np.uint16)


def test_reduce_exact_on_integer_rows():
    T, K, H = 16, 4, 64
    R = T * K
    X = ((np.arange(R)[:, None] * 7 + np.arange(H)[None, :]) % 64 - 32).astype(np.float32)
    rng = np.random.default_rng(0)
    pos = rng.permutation(R).reshape(T, K).astype(np.int32)
    pos[rng.random((T, K)) < 0.25] = -1
    w = np.exp2(-rng.integers(0, 4, size=(T, K))).astype(np.float32)
    got = oracle.reduce(oracle.BF16, _bits(X, torch.bfloat16), pos, w)
    assert np.array_equal(got, gather_sum(X, pos, w))


@pytest.mark.parametrize("dt,tdt", [(oracle.F16, torch.float16), (oracle.BF16, torch.bfloat16),
                                    (oracle.F32, torch.float32)])
@pytest.mark.parametrize("T,K,H", [(4, 2, 256), (16, 2, 512), (32, 8, 3072), (1, 8, 256),
                                   (8, 1, 256), (32, 8, 7168)])
def test_reduce_matches_gather_sum(dt, tdt, T, K, H):
    rng = np.random.default_rng(T * K + H)
    R = T * K
    Xf = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(tdt)
    X = Xf.float().numpy() if dt == oracle.F32 else Xf.view(torch.int16).numpy().view(np.uint16)
    pos = rng.permutation(R).reshape(T, K).astype(np.int32)
    pos[rng.random((T, K)) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    got = oracle.reduce(dt, X, pos, w)
    ref = gather_sum(Xf.float().numpy(), pos, w)
    assert np.max(np.abs(got - ref)) < 1e-5


def test_masked_rows_are_never_read():
    T, K, H = 3, 2, 8
    X = np.ones((7, H), np.float32)
    X[6] = np.nan          # the row a wrapped index -1 would read
    pos = np.array([[0, -1], [-1, -1], [5, 1]], np.int32)
    got = oracle.reduce(oracle.F32, X, pos, np.full((T, K), 0.5, np.float32))
    assert not np.any(np.isnan(got))
    assert got[:, 0].tolist() == [0.5, 0.0, 1.0]


def test_null_weights_equal_ones():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((40, 32)).astype(np.float32)
    pos = rng.permutation(40).reshape(10, 4).astype(np.int32)
    a = oracle.reduce(oracle.F32, X, pos, None)
    b = oracle.reduce(oracle.F32, X, pos, np.ones((10, 4), np.float32))
    assert np.array_equal(a, b)


def test_k1_is_a_scaled_gather():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((8, 16)).astype(np.float32)
    pos = rng.permutation(8).reshape(8, 1).astype(np.int32)
    w = rng.random((8, 1)).astype(np.float32)
    got = oracle.reduce(oracle.F32, X, pos, w)
    assert np.array_equal(got, (w * X[pos[:, 0]]).astype(np.float32))


def test_reduce_rejects_out_of_range_positions():
    X = np.zeros((4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.reduce(oracle.F32, X, np.array([[0, 4]], np.int32), None)


# ------------------------------------------------- scaled / FP8 variants ---
# (TileOPs-Metax PR #55, section 1: x_sf scales each routed slot's row, sf each
# token's output; FP8 E4M3 rows in and out.)

def gather_sum_scaled(X, pos, w, x_sf, sf):
    """float64 reference: sf[t] * sum_k w[t,k] * x_sf[pos] * X[pos] over pos >= 0."""
    T, K = pos.shape
    w = np.ones((T, K)) if w is None else w.astype(np.float64)
    xs = np.ones(X.shape[0]) if x_sf is None else x_sf.astype(np.float64)
    wk = w * xs[np.clip(pos, 0, None)] * (pos >= 0)
    y = np.einsum("tk,tkh->th", wk, np.asarray(X, np.float64)[np.clip(pos, 0, None)])
    return y if sf is None else y * sf.astype(np.float64)[:, None]


def _exact_case(seed, T=12, K=4, H=32):
    rng = np.random.default_rng(seed)
    R = T * K + 3
    X = rng.integers(-16, 17, size=(R, H)).astype(np.float32)
    pos = rng.permutation(R)[:T * K].reshape(T, K).astype(np.int32)
    pos[rng.random((T, K)) < 0.2] = -1
    w = np.exp2(-rng.integers(0, 3, size=(T, K))).astype(np.float32)
    x_sf = np.exp2(rng.integers(-2, 3, size=R)).astype(np.float32)
    sf = np.exp2(rng.integers(-3, 2, size=T)).astype(np.float32)
    return X, pos, w, x_sf, sf


def test_scaled_reduce_exact_with_power_of_two_scales():
    # Integer rows times powers of two: every product and partial sum is exact,
    # so the result must equal the float64 formula to the bit. A scale indexed
    # by slot or by token instead of by expanded row changes the answer.
    X, pos, w, x_sf, sf = _exact_case(7)
    got = oracle.reduce(oracle.F32, X, pos, w, x_sf=x_sf, sf=sf)
    assert np.array_equal(got, gather_sum_scaled(X, pos, w, x_sf, sf))
    by_slot = (w * x_sf[:pos.size].reshape(pos.shape)).astype(np.float32)
    assert not np.array_equal(got, gather_sum_scaled(X, pos, by_slot, None, sf))
    by_token = (w * x_sf[:pos.shape[0], None]).astype(np.float32)
    assert not np.array_equal(got, gather_sum_scaled(X, pos, by_token, None, sf))


def test_scaled_reduce_each_scale_alone():
    X, pos, w, x_sf, sf = _exact_case(8)
    base = oracle.reduce(oracle.F32, X, pos, w)
    only_sf = oracle.reduce(oracle.F32, X, pos, w, sf=sf)
    assert np.array_equal(only_sf, base * sf[:, None])
    only_xsf = oracle.reduce(oracle.F32, X, pos, w, x_sf=x_sf)
    assert np.array_equal(only_xsf, gather_sum_scaled(X, pos, w, x_sf, None))
    ones = oracle.reduce(oracle.F32, X, pos, w, x_sf=np.ones(X.shape[0], np.float32),
                         sf=np.ones(pos.shape[0], np.float32))
    assert np.array_equal(ones, base)


def test_scaled_reduce_uniform_x_sf_folds_into_weights():
    rng = np.random.default_rng(9)
    X = rng.standard_normal((30, 64)).astype(np.float32)
    pos = rng.permutation(30).reshape(10, 3).astype(np.int32)
    w = rng.random((10, 3)).astype(np.float32)
    c = np.float32(0.37)
    a = oracle.reduce(oracle.F32, X, pos, w, x_sf=np.full(30, c, np.float32))
    b = oracle.reduce(oracle.F32, X, pos, (w * c).astype(np.float32))
    assert np.array_equal(a, b)


def test_fp8_rows_reduce_to_the_decoded_sum():
    # FP8 rows: the reduce sees exactly the decoded values.
    rng = np.random.default_rng(10)
    T, K, H = 16, 4, 256
    R = T * K
    codes = rng.integers(0, 256, size=(R, H)).astype(np.uint8)
    codes[(codes & 0x7f) == 0x7f] = 0x38                  # no NaN codes
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    pos = rng.permutation(R).reshape(T, K).astype(np.int32)
    pos[rng.random((T, K)) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    x_sf = rng.random(R).astype(np.float32) + 0.5
    got = oracle.reduce(oracle.FP8, codes, pos, w, x_sf=x_sf)
    assert np.array_equal(got, oracle.reduce(oracle.F32, dec, pos, w, x_sf=x_sf))
    ref = gather_sum_scaled(dec, pos, w, x_sf, None)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
