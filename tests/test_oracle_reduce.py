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
