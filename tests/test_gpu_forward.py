"""The routed-MoE forward on the GPU against the oracle (same seeded inputs).

  * the tiny fp16 and mid-size bf16 workloads in full: every output element,
    plus the per-stage intermediates h and expert_out row by row;
  * small ragged shapes that span several column tiles and row groups, with
    masked slots, empty experts and experts that overflow one row block, at
    every supported block_m;
  * the DeepSeek-shaped decode / prefill / skewed workloads at full size, in
    the launch configuration the benchmark times: the decode workload on all
    512 tokens, the T = 4096 workloads on a token set that puts a checked row
    in every 32-row group of every scheduled row block of every active
    expert (both passes of the skewed workload's 256-row blocks included).
Outputs are pre-filled with NaN so an unwritten element fails the test.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import (ORACLE_DT, REL_L2_32, assert_close_16, cover_tokens, gpu_available,
                     metrics, storage)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _run(d, block_m=None):
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], E, block_m=block_m)
    ws, h, eo = mr.forward_workspace(tables, H, D, d["x"].dtype)
    h.fill_(float("nan"))
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y, workspace=ws)
    torch.cuda.synchronize()
    return tables, h, eo, y


def _oracle(d, tokens=None, want_pairs=True):
    dt = ORACLE_DT[d["x"].dtype]
    return oracle.moe_forward(dt, storage(d["x"]), storage(d["w_gate"]), storage(d["w_up"]),
                              storage(d["w_down"]), d["topk_ids"].cpu().numpy(),
                              d["topk_weights"].cpu().numpy(), tokens=tokens,
                              want_pairs=want_pairs)


def _check_pairs(tables, h, eo, hp, ep, K, token_index=None):
    """Sorted rows of h / expert_out against the oracle's per-slot values."""
    pos = tables.token_topk_to_pos.cpu().numpy()
    hg, eg = h.float().cpu().numpy(), eo.float().cpu().numpy()
    rows_h, rows_e, ref_h, ref_e = [], [], [], []
    tokens = range(hp.shape[0] // K) if token_index is None else token_index
    for i, t in enumerate(tokens):
        for k in range(K):
            p = pos[t * K + k]
            if p < 0:
                continue
            rows_h.append(hg[p]); ref_h.append(hp[i * K + k])
            rows_e.append(eg[p]); ref_e.append(ep[i * K + k])
    if not rows_h:
        return
    mh = metrics(np.stack(rows_h), np.stack(ref_h))
    me = metrics(np.stack(rows_e), np.stack(ref_e))
    assert not np.isnan(np.stack(rows_h)).any() and not np.isnan(np.stack(rows_e)).any()
    scale_h = max(1.0, float(np.abs(np.stack(ref_h)).max()))
    assert mh[1] <= 5e-3 and mh[0] <= 2e-2 * scale_h, ("h", mh)
    assert me[1] <= 5e-3 and me[0] <= 2e-2 * max(1.0, float(np.abs(np.stack(ref_e)).max())), ("eo", me)


@pytest.mark.parametrize("ci", [0, 1])
def test_forward_small_workloads_full(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    tables, h, eo, y = _run(d)
    y_ref, hp, ep = _oracle(d)
    got = y.float().cpu().numpy()
    assert_close_16(got, y_ref, cfg["name"])
    _check_pairs(tables, h, eo, hp, ep, cfg["K"])


def _custom(T, H, D, E, K, dtype, seed, mask=0.0, hot=None):
    cfg = dict(name="custom", dtype=dtype, T=T, H=H, D=D, E=E, K=K, renorm=True, zipf=False,
               seed=seed)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone()
    g = torch.Generator().manual_seed(seed)
    if hot is not None:     # send slot 0 of most tokens to one expert
        sel = torch.rand(T, generator=g) < 0.9
        col = ids[:, 0].cpu()
        col[sel] = hot
        # keep the K ids of a token distinct
        clash = (ids[:, 1:].cpu() == hot).any(dim=1) & sel
        col[clash] = ids[:, 0].cpu()[clash]
        ids[:, 0] = col.to(DEV)
    if mask:
        m = (torch.rand(T, K, generator=g) < mask).to(DEV)
        ids[m] = -1
    d["topk_ids"] = ids.contiguous()
    return d


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_forward_ragged(dtype, block_m):
    d = _custom(T=97, H=512, D=384, E=6, K=3, dtype=dtype, seed=11, mask=0.15, hot=2)
    tables, h, eo, y = _run(d, block_m=block_m)
    sizes = tables.group_sizes.cpu().numpy()
    assert sizes.max() > 64          # an expert spans more than one block at small block_m
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "ragged")
    _check_pairs(tables, h, eo, hp, ep, 3)


@pytest.mark.parametrize("block_m", [128, 256])
def test_forward_wide_blocks(block_m):
    """Prefill-sized blocks: full 256-row blocks (two passes of 4 row groups),
    a 193..224-row tail block, one-pass blocks of up to 6 row groups, and
    reductions of 8 and 6 chunks (the pipeline tail with and without a full
    group of steps)."""
    d = _custom(T=600, H=512, D=384, E=4, K=2, dtype="bf16", seed=21, mask=0.05, hot=1)
    tables, h, eo, y = _run(d, block_m=block_m)
    sizes = tables.group_sizes.cpu().numpy()
    assert sizes.max() > 2 * 256 and (sizes % 256).max() > 0
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "wide blocks")
    _check_pairs(tables, h, eo, hp, ep, 2)


@pytest.mark.parametrize("block_m", [16, 32])
def test_forward_deep_pipeline_tails(block_m):
    """Decode-sized blocks with reductions long enough for the deepest
    pipelines (gate/up: 24 chunks of 64, full groups of steps and a tail;
    down: 20 chunks) and ragged rows."""
    d = _custom(T=70, H=1536, D=1280, E=5, K=3, dtype="bf16", seed=16, mask=0.1, hot=1)
    tables, h, eo, y = _run(d, block_m=block_m)
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "deep pipeline")
    _check_pairs(tables, h, eo, hp, ep, 3)


def test_forward_empty_experts_and_all_masked_tokens():
    d = _custom(T=40, H=256, D=128, E=16, K=2, dtype="bf16", seed=12)
    ids = d["topk_ids"]
    ids[ids >= 8] = 3                 # experts 8..15 get no rows
    ids[5] = -1                       # token 5 fully masked
    ids[:, 1] = torch.where(ids[:, 1] == ids[:, 0], -1, ids[:, 1])
    d["topk_ids"] = ids.contiguous()
    tables, h, eo, y = _run(d, block_m=16)
    assert (tables.group_sizes.cpu().numpy()[8:] == 0).all()
    y_ref, hp, ep = _oracle(d)
    assert torch.all(y[5] == 0)
    assert_close_16(y.float().cpu().numpy(), y_ref, "empty experts")
    _check_pairs(tables, h, eo, hp, ep, 2)


def test_forward_single_token_single_expert():
    d = _custom(T=1, H=256, D=128, E=1, K=1, dtype="bf16", seed=13)
    tables, h, eo, y = _run(d)
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "T=1")


def test_forward_stages_match_forward():
    mr = _mr()
    d = _custom(T=64, H=512, D=256, E=8, K=2, dtype="bf16", seed=14)
    tables, h, eo, y = _run(d)
    h2 = mr.moe_expert_gate_up(d["x"], d["w_gate"], d["w_up"], tables)
    eo2 = mr.moe_expert_down(h2, d["w_down"], tables)
    y2 = mr.moe_reduce_fused(eo2, tables.token_topk_to_pos.view(64, 2), tables.topk_weights.view(64, 2))
    n = int(tables.group_sizes.sum())
    assert torch.equal(h2[:n], h[:n]) and torch.equal(eo2[:n], eo[:n]) and torch.equal(y2, y)


def test_forward_argument_errors():
    mr = _mr()
    d = _custom(T=8, H=256, D=128, E=4, K=2, dtype="bf16", seed=15)
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 4)
    with pytest.raises(mr.MoeError) as ei:       # w_up of another shape
        mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"][:, :64].contiguous(), d["w_down"], tables)
    assert ei.value.status == 2
    with pytest.raises(mr.MoeError) as ei:       # float64 inputs
        mr.moe_routed_forward(d["x"].double(), d["w_gate"].double(), d["w_up"].double(),
                              d["w_down"].double(), tables)
    assert ei.value.status == 3
    with pytest.raises(mr.MoeError) as ei:       # mixed dtypes
        mr.moe_routed_forward(d["x"], d["w_gate"].float(), d["w_up"], d["w_down"], tables)
    assert ei.value.status == 3
    with pytest.raises(mr.MoeError) as ei:       # weights of the wrong dtype
        mr.moe_dispatch(d["topk_ids"], d["topk_weights"].half(), 4)
    assert ei.value.status == 3


# ------------------------------------------------------------- fp32 path ---

@pytest.mark.parametrize("ci", [0, 1])
def test_forward_fp32_debug_path(ci):
    # The fp32 build of the forward against the oracle's fp32 storage (no
    # intermediate rounding): rel-L2 <= 1e-4.
    cfg = dict(S.CONFIGS[ci], dtype="f32")
    d = S.make_moe_inputs(cfg, device=DEV)
    tables, h, eo, y = _run(d)
    y_ref, hp, ep = _oracle(d)
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    mabs, rel = metrics(got, y_ref)
    assert rel <= REL_L2_32, (mabs, rel)
    _check_pairs(tables, h, eo, hp, ep, cfg["K"])


@pytest.mark.parametrize("block_m", [16, 64, 256])
def test_forward_fp32_ragged(block_m):
    d = _custom(T=97, H=512, D=384, E=6, K=3, dtype="f32", seed=21, mask=0.15, hot=2)
    tables, h, eo, y = _run(d, block_m=block_m)
    y_ref, hp, ep = _oracle(d)
    mabs, rel = metrics(y.cpu().numpy(), y_ref)
    assert rel <= REL_L2_32, (mabs, rel)


# ------------------------------------------------------------ full sizes ---

def _sampled_oracle(d, tokens):
    """The oracle on `tokens`, given only the experts those tokens use."""
    ids = d["topk_ids"].cpu().numpy()[tokens]
    used = np.unique(ids[ids >= 0])
    remap = np.full(d["E"], -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sel = torch.from_numpy(used).long().to(DEV)
    dt = ORACLE_DT[d["x"].dtype]
    sub_ids = np.where(ids >= 0, remap[np.maximum(ids, 0)], -1).astype(np.int32)
    return oracle.moe_forward(dt, storage(d["x"][torch.from_numpy(tokens).long().to(DEV)]),
                              storage(d["w_gate"][sel]), storage(d["w_up"][sel]),
                              storage(d["w_down"][sel]), sub_ids,
                              d["topk_weights"].cpu().numpy()[tokens], want_pairs=True)


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_forward_full_size_sampled(ci):
    mr = _mr()
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"])
    tables, h, eo, y = _run(d, block_m=block_m)
    assert not torch.isnan(y).any()
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m)
    y_ref, hp, ep = _sampled_oracle(d, tokens)
    assert_close_16(y.float().cpu().numpy()[tokens], y_ref, cfg["name"])
    _check_pairs(tables, h, eo, hp, ep, cfg["K"], token_index=list(tokens))
    del d, h, eo, y, tables
    torch.cuda.empty_cache()
