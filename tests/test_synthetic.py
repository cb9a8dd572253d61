"""The seeded input generator: reproducibility and the workloads' stated structure."""
import math

import numpy as np
import pytest
import torch

import synthetic as S


def test_counter_rng_matches_python_reference():
    b = S.bits64(7, 3, 100, 64)
    key = S.stream_key(7, 3)
    ref = [S.mix64_py(key + (i + 1) * S.GOLDEN) for i in range(100, 164)]
    assert [int(v) & S.MASK64 for v in b.tolist()] == ref


def test_splitmix64_known_value():
    # SplitMix64 seeded with 0: the first output is 0xE220A8397B1DCDAF.
    assert S.mix64_py(S.GOLDEN) == 0xE220A8397B1DCDAF


def test_values_do_not_depend_on_chunking(monkeypatch):
    a = S.normal((1000,), 1.0, 3, 1, torch.float32)
    monkeypatch.setattr(S, "_CHUNK", 77)
    b = S.normal((1000,), 1.0, 3, 1, torch.float32)
    assert torch.equal(a, b)


def test_normal_moments():
    z = S.normal((1 << 20,), 1.0, 11, 2, torch.float32).double()
    assert abs(z.mean().item()) < 5e-3
    assert abs(z.std().item() - 1.0) < 5e-3
    u = S.uniform(11, 3, 0, 1 << 20)
    assert 0.0 < u.min().item() and u.max().item() < 1.0


def test_routing_ties_go_to_lower_index():
    x = torch.ones(2, 4)
    router = torch.zeros(6, 4)   # all logits equal
    ids, w = S.route(x, router, 3, renorm=False)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert torch.allclose(w, torch.full((2, 3), 1.0 / 6))


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_workload_routing_shape(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, weights=False)
    ids, w = d["topk_ids"], d["topk_weights"]
    assert ids.shape == (cfg["T"], cfg["K"]) and ids.dtype == torch.int32
    assert int(ids.min()) >= 0 and int(ids.max()) < cfg["E"]
    assert all(len(set(r)) == cfg["K"] for r in ids.tolist())
    if cfg["renorm"]:
        assert torch.allclose(w.sum(-1), torch.ones(cfg["T"]), atol=1e-6)
    else:
        assert float(w.sum(-1).max()) < 1.0


def test_skewed_workload_has_cold_and_hot_experts():
    cfg = S.CONFIGS[4]
    d = S.make_moe_inputs(cfg, weights=False)
    cnt = torch.bincount(d["topk_ids"].view(-1).long(), minlength=cfg["E"])
    assert int((cnt == 0).sum()) >= 1
    assert int(cnt.max()) > 1000


def test_reduce_inputs_structure():
    d = S.make_reduce_inputs(64, 8, 256, seed=4)
    pos = d["token_topk_to_pos"].view(-1)
    P = 64 * 8
    assert int((pos == -1).sum()) == math.floor(0.1 * P)
    kept = pos[pos >= 0]
    assert kept.unique().numel() == kept.numel()
    assert torch.allclose(d["topk_weights"].sum(-1), torch.ones(64), atol=1e-6)
    assert d["expert_out"].shape == (P, 256) and d["expert_out"].dtype == torch.bfloat16


def test_weights_std_follows_fan_in():
    cfg = dict(S.CONFIGS[1])
    d = S.make_moe_inputs(cfg, T=4)
    assert abs(d["w_gate"].float().std().item() * math.sqrt(cfg["H"]) - 1) < 0.01
    assert abs(d["w_down"].float().std().item() * math.sqrt(cfg["D"]) - 1) < 0.01
