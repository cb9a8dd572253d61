"""The forward with the routing weight in the down GEMM's epilogue
(moe_expert_down_weighted / moe_routed_forward_weighted) on the GPU against
the oracle's weighted-down forward, on the same seeded inputs.

  * the tiny fp16 and mid-size bf16 workloads in full, with the weighted
    expert_out rows checked row by row;
  * ragged shapes with masked slots and an overflowing expert at every
    block_m (both GEMM kernels), prefill-sized blocks, the fp32 path;
  * exact properties of the kernels: with power-of-two weights every
    weighted row is w times the unweighted row and y equals the
    weighted-combine forward bit for bit; with weights NULL at dispatch the
    two forward forms give identical bits; the separate calls equal the
    one-call forward;
  * the DeepSeek-shaped decode / prefill workloads at full size, in the
    launch configuration the benchmark times, on sampled tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import (ORACLE_DT, REL_L2_32, assert_close_16, cover_tokens, gpu_available,
                     metrics, storage)
from test_gpu_forward import _custom

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _run(d, block_m=None, weighted=True, weights="given"):
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tw = d["topk_weights"] if weights == "given" else None
    tables = mr.moe_dispatch(d["topk_ids"], tw, E, block_m=block_m)
    ws, h, eo = mr.forward_workspace(tables, H, D, d["x"].dtype)
    h.fill_(float("nan"))
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y, workspace=ws,
                          weighted_down=weighted)
    torch.cuda.synchronize()
    return tables, h, eo, y


def _oracle(d, tokens=None, sub=None):
    dt = ORACLE_DT[d["x"].dtype]
    if sub is None:
        args = [storage(d[n]) for n in ("x", "w_gate", "w_up", "w_down")]
        ids = d["topk_ids"].cpu().numpy()
        w = d["topk_weights"].cpu().numpy()
    else:
        args, ids, w = sub
    return oracle.moe_forward(dt, *args, ids, w, tokens=tokens, want_pairs=True,
                              weighted_down=True)


def _check_rows(tables, eo, ep, K, tokens, tol_rel=5e-3):
    pos = tables.token_topk_to_pos.cpu().numpy()
    eg = eo.float().cpu().numpy()
    got, ref = [], []
    for i, t in enumerate(tokens):
        for k in range(K):
            p = pos[t * K + k]
            if p >= 0:
                got.append(eg[p])
                ref.append(ep[i * K + k])
    got, ref = np.stack(got), np.stack(ref)
    assert not np.isnan(got).any()
    mabs, rel = metrics(got, ref)
    assert rel <= tol_rel and mabs <= 2e-2 * max(1.0, float(np.abs(ref).max())), (mabs, rel)


@pytest.mark.parametrize("ci", [0, 1])
def test_weighted_forward_small_workloads_full(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    tables, h, eo, y = _run(d)
    y_ref, _, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, cfg["name"])
    _check_rows(tables, eo, ep, cfg["K"], range(cfg["T"]))


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_forward_ragged(dtype, block_m):
    d = _custom(T=97, H=512, D=384, E=6, K=3, dtype=dtype, seed=31, mask=0.15, hot=2)
    tables, h, eo, y = _run(d, block_m=block_m)
    assert tables.group_sizes.cpu().numpy().max() > 64
    y_ref, _, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "ragged weighted")
    _check_rows(tables, eo, ep, 3, range(97))


@pytest.mark.parametrize("block_m", [128, 256])
def test_weighted_forward_wide_blocks(block_m):
    d = _custom(T=600, H=512, D=384, E=4, K=2, dtype="bf16", seed=32, mask=0.05, hot=1)
    tables, h, eo, y = _run(d, block_m=block_m)
    assert tables.group_sizes.cpu().numpy().max() > 2 * 256
    y_ref, _, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "wide weighted")
    _check_rows(tables, eo, ep, 2, range(600))


@pytest.mark.parametrize("block_m", [16, 256])
def test_weighted_forward_fp32(block_m):
    d = _custom(T=97, H=512, D=384, E=6, K=3, dtype="f32", seed=33, mask=0.15, hot=2)
    tables, h, eo, y = _run(d, block_m=block_m)
    y_ref, _, ep = _oracle(d)
    mabs, rel = metrics(y.cpu().numpy(), y_ref)
    assert not np.isnan(y.cpu().numpy()).any() and rel <= REL_L2_32, (mabs, rel)
    _check_rows(tables, eo, ep, 3, range(97), tol_rel=REL_L2_32)


@pytest.mark.parametrize("block_m", [32, 64, 256])
def test_power_of_two_weights_scale_rows_exactly(block_m):
    d = _custom(T=200, H=512, D=256, E=5, K=2, dtype="bf16", seed=34, mask=0.1, hot=0)
    g = torch.Generator().manual_seed(34)
    d["topk_weights"] = (2.0 ** -torch.randint(0, 5, d["topk_weights"].shape, generator=g)).float().to(DEV)
    t0, _, e0, y0 = _run(d, block_m=block_m, weighted=False)
    t1, _, e1, y1 = _run(d, block_m=block_m, weighted=True)
    n = int(t0.group_sizes.sum())
    w = t0.sorted_weight[:n].view(-1, 1)
    assert torch.equal(e1[:n].float(), e0[:n].float() * w)
    assert torch.equal(y0, y1)


def test_null_weights_forms_identical():
    d = _custom(T=64, H=512, D=256, E=8, K=2, dtype="bf16", seed=35, mask=0.1)
    _, _, e0, y0 = _run(d, weighted=False, weights=None)
    _, _, e1, y1 = _run(d, weighted=True, weights=None)
    assert torch.equal(y0, y1)


def test_weighted_stages_match_forward():
    mr = _mr()
    d = _custom(T=64, H=512, D=256, E=8, K=2, dtype="bf16", seed=36)
    tables, h, eo, y = _run(d)
    h2 = mr.moe_expert_gate_up(d["x"], d["w_gate"], d["w_up"], tables)
    eo2 = mr.moe_expert_down_weighted(h2, d["w_down"], tables)
    y2 = mr.moe_reduce_fused(eo2, tables.token_topk_to_pos.view(64, 2), None)
    n = int(tables.group_sizes.sum())
    assert torch.equal(eo2[:n], eo[:n]) and torch.equal(y2, y)


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_weighted_forward_full_size_sampled(ci):
    mr = _mr()
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"])
    tables, h, eo, y = _run(d, block_m=block_m)
    assert not torch.isnan(y).any()
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m)
    ids = d["topk_ids"].cpu().numpy()[tokens]
    used = np.unique(ids[ids >= 0])
    remap = np.full(d["E"], -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sel = torch.from_numpy(used).long().to(DEV)
    sub = ([storage(d["x"][torch.from_numpy(tokens).long().to(DEV)])]
           + [storage(d[n][sel]) for n in ("w_gate", "w_up", "w_down")],
           np.where(ids >= 0, remap[np.maximum(ids, 0)], -1).astype(np.int32),
           d["topk_weights"].cpu().numpy()[tokens])
    y_ref, _, ep = _oracle(d, sub=sub)
    assert_close_16(y.float().cpu().numpy()[tokens], y_ref, cfg["name"])
    _check_rows(tables, eo, ep, cfg["K"], list(tokens))
    del d, h, eo, y, tables
    torch.cuda.empty_cache()
