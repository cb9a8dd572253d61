"""Pins for the oracle's routed-MoE forward (CPU only).

  * a dense float64 brute force with no dispatch at all,
        y[t] = sum_k w[t,k] * Wd_e (SiLU(Wg_e x_t) * (Wu_e x_t)),  e = ids[t,k],
    written with numpy matrix products over whole expert matrices, against
    the oracle in fp32 storage (no intermediate rounding);
  * closed forms: zero gate weights, identity weights, the single-expert
    SwiGLU MLP (K = 1, w = 1), all slots masked, linearity in the weights,
    token-permutation equivariance;
  * a hand-built case where SiLU saturates so every value is exact and the
    16-bit rounding of h and of expert_out (ties to even) decides the result.
"""
import numpy as np
import pytest
import torch

import oracle


def dense_brute_force(x, wg, wu, wd, ids, w):
    x, wg, wu, wd = (np.asarray(a, np.float64) for a in (x, wg, wu, wd))
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        for k in range(ids.shape[1]):
            e = ids[t, k]
            if e < 0:
                continue
            g = wg[e] @ x[t]
            u = wu[e] @ x[t]
            h = g / (1.0 + np.exp(-g)) * u
            y[t] += float(w[t, k]) * (wd[e] @ h)
    return y


def _rand(shape, scale, rng):
    # values exactly representable in bf16, so fp32 storage holds them exactly
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).float().numpy()


def _case(T, H, D, E, K, seed, mask=0.0):
    rng = np.random.default_rng(seed)
    x = _rand((T, H), 1.0, rng)
    wg = _rand((E, D, H), H ** -0.5, rng)
    wu = _rand((E, D, H), H ** -0.5, rng)
    wd = _rand((E, H, D), D ** -0.5, rng)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    if mask:
        ids[rng.random((T, K)) < mask] = -1
    w = rng.random((T, K)).astype(np.float32)
    return x, wg, wu, wd, ids, w


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


@pytest.mark.parametrize("T,H,D,E,K,mask", [(16, 64, 32, 4, 2, 0.0), (7, 32, 48, 3, 1, 0.0),
                                             (9, 64, 16, 4, 3, 0.3), (1, 8, 8, 1, 1, 0.0)])
def test_forward_matches_dense_brute_force(T, H, D, E, K, mask):
    x, wg, wu, wd, ids, w = _case(T, H, D, E, K, seed=T + H + D, mask=mask)
    got = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w)
    ref = dense_brute_force(x, wg, wu, wd, ids, w)
    assert _rel(got, ref) < 1e-5
    assert np.max(np.abs(got - ref)) < 1e-5 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("dt,tdt", [(oracle.BF16, torch.bfloat16), (oracle.F16, torch.float16)])
def test_forward_mirror_close_to_brute_force_with_rounding(dt, tdt):
    x, wg, wu, wd, ids, w = _case(12, 64, 32, 4, 2, seed=5)
    store = {"bits": lambda a: torch.from_numpy(a).to(tdt).view(torch.int16).numpy().view(np.uint16)}
    got = oracle.moe_forward(dt, *(store["bits"](a) for a in (x, wg, wu, wd)), ids, w)
    xs, gs, us, ds = (torch.from_numpy(a).to(tdt).double().numpy() for a in (x, wg, wu, wd))
    rnd = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(tdt).double().numpy()
    ref = np.zeros_like(xs)
    for t in range(xs.shape[0]):
        for k in range(ids.shape[1]):
            e = ids[t, k]
            g, u = gs[e] @ xs[t], us[e] @ xs[t]
            h = rnd(g / (1 + np.exp(-g)) * u)
            ref[t] += float(w[t, k]) * rnd(ds[e] @ h)
    assert _rel(got, ref) < 2e-3


def test_zero_gate_gives_zero():
    x, wg, wu, wd, ids, w = _case(8, 32, 16, 3, 2, seed=1)
    got = oracle.moe_forward(oracle.F32, x, np.zeros_like(wg), wu, wd, ids, w)
    assert np.all(got == 0.0)


def test_identity_weights():
    # H = D, Wg = Wu = Wd = I  =>  y[t] = (sum_k w[t,k]) * SiLU(x_t) * x_t
    T, H, E, K = 6, 16, 2, 2
    rng = np.random.default_rng(2)
    x = _rand((T, H), 1.0, rng)
    eye = np.broadcast_to(np.eye(H, dtype=np.float32), (E, H, H)).copy()
    ids = np.array([[0, 1]] * T, np.int32)
    w = np.full((T, K), 0.5, np.float32)
    got = oracle.moe_forward(oracle.F32, x, eye, eye, eye, ids, w)
    xd = x.astype(np.float64)
    ref = xd / (1 + np.exp(-xd)) * xd
    assert np.max(np.abs(got - ref)) < 1e-6


def test_single_expert_swiglu_mlp():
    # E = 1, K = 1, w = 1: the plain SwiGLU MLP Wd (SiLU(Wg x) * (Wu x)) per token
    x, wg, wu, wd, _, _ = _case(10, 32, 24, 1, 1, seed=3)
    ids = np.zeros((10, 1), np.int32)
    w = np.ones((10, 1), np.float32)
    got = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w)
    xd, gd, ud, dd = (a.astype(np.float64) for a in (x, wg[0], wu[0], wd[0]))
    g, u = xd @ gd.T, xd @ ud.T
    ref = (g / (1 + np.exp(-g)) * u) @ dd.T
    assert _rel(got, ref) < 1e-5


def test_all_masked_gives_zero():
    x, wg, wu, wd, ids, w = _case(5, 16, 16, 2, 2, seed=4)
    got = oracle.moe_forward(oracle.F32, x, wg, wu, wd, np.full_like(ids, -1), w)
    assert np.all(got == 0.0)


def test_linearity_in_routing_weights():
    x, wg, wu, wd, ids, w = _case(8, 32, 16, 4, 2, seed=6)
    y1 = oracle.moe_forward(oracle.BF16, *(torch.from_numpy(a).to(torch.bfloat16).view(torch.int16)
                                          .numpy().view(np.uint16) for a in (x, wg, wu, wd)), ids, w)
    y2 = oracle.moe_forward(oracle.BF16, *(torch.from_numpy(a).to(torch.bfloat16).view(torch.int16)
                                          .numpy().view(np.uint16) for a in (x, wg, wu, wd)), ids, 2 * w)
    assert np.array_equal(y2, 2 * y1)   # scaling by two is exact in fp32


def test_token_permutation_equivariance():
    x, wg, wu, wd, ids, w = _case(9, 32, 16, 4, 2, seed=7)
    perm = np.random.default_rng(0).permutation(9)
    y = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w)
    yp = oracle.moe_forward(oracle.F32, x[perm], wg, wu, wd, ids[perm], w[perm])
    assert np.array_equal(yp, y[perm])


def test_token_subset_and_pairs_agree_with_full():
    x, wg, wu, wd, ids, w = _case(11, 32, 16, 4, 3, seed=8, mask=0.2)
    y = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w)
    sub = np.array([10, 0, 5], np.int32)
    ys, hp, ep = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w, tokens=sub, want_pairs=True)
    assert np.array_equal(ys, y[sub])
    for i, t in enumerate(sub):
        for k in range(3):
            e = ids[t, k]
            if e < 0:
                assert np.all(hp[i * 3 + k] == 0) and np.all(ep[i * 3 + k] == 0)
                continue
            h, eo = oracle.expert_pair(oracle.F32, x, wg, wu, wd, t, e)
            assert np.array_equal(h, hp[i * 3 + k]) and np.array_equal(eo, ep[i * 3 + k])


@pytest.mark.parametrize("dt,tdt,g_w,step,h_exp,eo_exp,y_exp", [
    # bf16: g = 256 (SiLU(256) == 256 in fp32), u_j = 1 + (j+1) 2^-9, so
    # SiLU(g) u_j = 256.5, 257, 257.5, 258 -> bf16 (ulp 2): 256, 256 (tie->even),
    # 258, 258. expert_out: [h_0, (sum h)/2 = 514 -> tie -> 512]; y = eo / 4.
    (oracle.BF16, torch.bfloat16, 128.0, 2.0 ** -9, [256, 256, 258, 258], [256, 512], [64, 128]),
    # fp16: g = 2048, u_j = 1 + (j+1) 2^-12: 2048.5, 2049, 2049.5, 2050 ->
    # fp16 (ulp 2): 2048, 2048, 2050, 2050; (sum h)/2 = 4098 -> tie -> 4096.
    (oracle.F16, torch.float16, 1024.0, 2.0 ** -12, [2048, 2048, 2050, 2050], [2048, 4096],
     [512, 1024]),
])
def test_mirror_rounding_closed_form(dt, tdt, g_w, step, h_exp, eo_exp, y_exp):
    D = 4
    x = np.array([[1.0, 1.0]], np.float32)
    wg = np.array([[[g_w, g_w]] * D], np.float32)
    wu = np.array([[[1.0, (j + 1) * step] for j in range(D)]], np.float32)
    wd = np.array([[[1.0, 0.0, 0.0, 0.0], [0.5, 0.5, 0.5, 0.5]]], np.float32)
    bits = lambda a: torch.from_numpy(a).to(tdt).view(torch.int16).numpy().view(np.uint16)
    for a in (x, wg, wu, wd):   # every input is exactly representable
        assert np.array_equal(torch.from_numpy(a).to(tdt).float().numpy(), a)
    ids = np.zeros((1, 1), np.int32)
    w = np.full((1, 1), 0.25, np.float32)
    y, hp, ep = oracle.moe_forward(dt, bits(x), bits(wg), bits(wu), bits(wd), ids, w,
                                   want_pairs=True)
    assert hp[0].tolist() == h_exp
    assert ep[0].tolist() == eo_exp
    assert y[0].tolist() == y_exp
    # Without the intermediate rounding (fp32 storage) the exact values appear.
    y32, hp32, ep32 = oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w, want_pairs=True)
    assert hp32[0].tolist() == [h_exp[0] + 0.5, h_exp[0] + 1.0, h_exp[0] + 1.5, h_exp[0] + 2.0]
    assert ep32[0, 1] == sum(hp32[0]) / 2


def test_forward_rejects_bad_ids():
    x, wg, wu, wd, ids, w = _case(3, 16, 16, 2, 1, seed=9)
    ids[1, 0] = 2
    with pytest.raises(ValueError):
        oracle.moe_forward(oracle.F32, x, wg, wu, wd, ids, w)
