"""Pins for the oracle's router gate (CPU only).

The gate is the step in front of the routed experts, specified by the
routed-MoE workload recipes: fp32 softmax of x . Wr^T, top-k by score with
ties to the lower index, weights = the selected scores, optionally
renormalised. What pins the oracle, independently of its own code:
  * logits exact on integer-valued inputs (every fp32 partial sum exact), so
    a transposed operand or a dropped term fails;
  * logits within the fp32 accumulation bound of a float64 matmul;
  * selection equal to a stable sort (numpy) of its own logits, ties to the
    lower index on duplicated router rows;
  * scores equal to a float64 softmax of its logits; K = E without
    renormalisation sums to 1; renormalised weights sum to 1; the two-expert
    case is the logistic function of the logit difference;
  * a logit bias adds in one fp32 addition (logits = unbiased + bias);
  * agreement with the workload recipe's own router (float64 logits, torch
    softmax and sort) except at near-ties of the logits, including the
    skewed recipe's Zipf bias.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _stable_topk(logits, K):
    E = logits.shape[1]
    idx = np.broadcast_to(np.arange(E), logits.shape)
    out = np.empty((logits.shape[0], K), np.int64)
    for t in range(logits.shape[0]):
        order = np.lexsort((idx[t], -logits[t].astype(np.float64)))
        out[t] = order[:K]
    return out


def test_gate_logits_exact_on_integer_inputs():
    rng = np.random.default_rng(0)
    T, H, E = 9, 64, 12
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    wr = rng.integers(-8, 9, size=(E, H)).astype(np.float32)
    g = oracle.gate(oracle.BF16, _bf16(x), wr, K=3, renorm=False)
    exact = x.astype(np.int64) @ wr.astype(np.int64).T
    assert np.array_equal(g["logits"], exact.astype(np.float32))


def test_gate_logits_within_fp32_bound_of_float64():
    rng = np.random.default_rng(1)
    T, H, E = 16, 2048, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    g = oracle.gate(oracle.F32, x, wr, K=4, renorm=True)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    bound = H * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(wr).astype(np.float64).T)
    assert np.all(np.abs(g["logits"] - ref) <= bound)


def test_gate_selection_is_stable_sort_of_logits():
    rng = np.random.default_rng(2)
    T, H, E, K = 32, 256, 64, 8
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    g = oracle.gate(oracle.BF16, _bf16(x), wr, K=K, renorm=True)
    assert np.array_equal(g["ids"], _stable_topk(g["logits"], K))


def test_gate_ties_go_to_lower_index():
    T, H, E = 4, 64, 6
    x = np.ones((T, H), np.float32)
    wr = np.zeros((E, H), np.float32)
    wr[1] = 0.5
    wr[4] = 0.5          # identical to row 1: the lower index comes first
    wr[2] = 0.25
    wr[5] = 0.25
    g = oracle.gate(oracle.F32, x, wr, K=4, renorm=False)
    assert np.array_equal(g["ids"], np.tile([1, 4, 2, 5], (T, 1)))
    assert np.all(g["weights"][:, 0] == g["weights"][:, 1])


def test_gate_scores_are_softmax_of_logits():
    rng = np.random.default_rng(3)
    T, H, E, K = 16, 128, 40, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    g = oracle.gate(oracle.F32, x, wr, K=K, renorm=False)
    l = g["logits"].astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = np.take_along_axis(p, g["ids"].astype(np.int64), axis=1)
    assert np.allclose(g["weights"], ref, rtol=2e-6, atol=0)
    # renormalised: the selected scores over their sum
    gr = oracle.gate(oracle.F32, x, wr, K=K, renorm=True)
    assert np.array_equal(gr["ids"], g["ids"])
    assert np.allclose(gr["weights"], ref / ref.sum(axis=1, keepdims=True), rtol=2e-6, atol=0)
    assert np.allclose(gr["weights"].sum(axis=1), 1.0, rtol=0, atol=2e-6)


def test_gate_full_softmax_sums_to_one():
    rng = np.random.default_rng(4)
    T, H, E = 8, 64, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    g = oracle.gate(oracle.F32, x, wr, K=E, renorm=False)
    assert np.allclose(g["weights"].sum(axis=1), 1.0, rtol=0, atol=4e-6)
    assert np.all(np.diff(g["weights"], axis=1) <= 0)          # sorted by score


def test_gate_two_experts_is_logistic():
    rng = np.random.default_rng(5)
    T, H = 64, 32
    x = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    wr = rng.integers(-2, 3, size=(2, H)).astype(np.float32) / 8.0
    g = oracle.gate(oracle.F32, x, wr, K=1, renorm=False)
    d = (x.astype(np.float64) @ (wr[0] - wr[1]).astype(np.float64))   # exact
    p0 = 1.0 / (1.0 + np.exp(-d))
    top = np.where(d >= 0, 0, 1)
    assert np.array_equal(g["ids"][:, 0], top)
    assert np.allclose(g["weights"][:, 0], np.maximum(p0, 1 - p0), rtol=2e-6, atol=0)


def test_gate_bias_adds_once():
    rng = np.random.default_rng(6)
    T, H, E = 8, 128, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 3).astype(np.float32)
    g0 = oracle.gate(oracle.F32, x, wr, K=4, renorm=True)
    g1 = oracle.gate(oracle.F32, x, wr, K=4, renorm=True, bias=b)
    assert np.array_equal(g1["logits"], (g0["logits"] + b[None, :]).astype(np.float32))
    assert np.array_equal(g1["ids"], _stable_topk(g1["logits"], 4))


@pytest.mark.parametrize("ci,T", [(0, None), (1, None), (4, 256)])
def test_gate_matches_workload_recipe_router(ci, T):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device="cpu", weights=False, T=T)
    T = d["T"]
    x = d["x"]
    dt = {torch.float16: oracle.F16, torch.bfloat16: oracle.BF16}[x.dtype]
    xs = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    bias = S.zipf_bias(cfg["E"]).numpy() if cfg.get("zipf") else None
    g = oracle.gate(dt, xs, d["router"].numpy(), K=cfg["K"], renorm=cfg["renorm"], bias=bias)
    ids_ref = d["topk_ids"].numpy()
    l64 = (x.to(torch.float64) @ d["router"].to(torch.float64).t()).numpy()
    if bias is not None:
        l64 = l64 + bias.astype(np.float64)
    bad = np.where((g["ids"] != ids_ref).any(axis=1))[0]
    # the recipe ranks float64 logits; the oracle ranks fp32 fma-chain logits:
    # they may only disagree where two candidates' logits are within rounding
    assert len(bad) <= max(1, T // 100)
    for t in bad:
        l = np.sort(l64[t])[::-1][: cfg["K"] + 1]
        assert np.min(np.abs(np.diff(l))) < 1e-5
    ok = np.setdiff1d(np.arange(T), bad)
    # weights: exp turns a logit difference dl into a relative weight
    # difference of about dl; the fp32 chain is within H*2^-24*sum|x w| of
    # the float64 logit, and w = exp(l_k - m) / Z involves three logits.
    xa = np.abs(x.to(torch.float64).numpy())
    dl = cfg["H"] * 2.0 ** -24 * (xa @ np.abs(d["router"].numpy().astype(np.float64)).T)
    rtol = 3 * dl.max() + 2e-6
    assert np.allclose(g["weights"][ok], d["topk_weights"].numpy()[ok], rtol=rtol, atol=1e-9)
