"""The fused expert kernel (gate/up and down of a row block in one
workgroup, h kept in LDS) on the GPU:

  * against the oracle (same seeded inputs): the tiny and mid-size
    workloads in full, ragged shapes with masked slots, empty experts and a
    hot expert at block_m 16 and 32, reductions long enough for the deep
    pipelines and short enough for the depth-2 form, d_expert at its 2048
    limit, and the DeepSeek-shaped decode workload on a token set that puts
    a checked row in every scheduled row block;
  * bit for bit against the two-kernel path (moe_expert_gate_up then
    moe_expert_down, and moe_routed_forward): both round h the same way and
    sum every dot product in the same order;
  * the argument checks (block_m above 32, d_expert above the LDS limit,
    fp32, a short workspace).
Outputs are pre-filled with NaN so an unwritten element fails the test.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import ORACLE_DT, assert_close_16, cover_tokens, gpu_available, metrics, storage

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _custom(T, H, D, E, K, dtype, seed, mask=0.0, hot=None):
    cfg = dict(name="custom", dtype=dtype, T=T, H=H, D=D, E=E, K=K, renorm=True, zipf=False,
               seed=seed)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone().cpu()
    g = torch.Generator().manual_seed(seed)
    if hot is not None:     # slot 0 of most tokens to one expert, ids of a token distinct
        sel = torch.rand(T, generator=g) < 0.9
        clash = (ids[:, 1:] == hot).any(dim=1)
        ids[sel & ~clash, 0] = hot
    if mask:
        ids[torch.rand(T, K, generator=g) < mask] = -1
    d["topk_ids"] = ids.to(DEV).contiguous()
    return d


def _run_both(d, block_m):
    """The fused forward and the two-kernel forward on the same tables."""
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], E, block_m=block_m)
    ws, eo = mr.fused_workspace(tables, H, d["x"].dtype)
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward_fused(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y,
                                workspace=ws)
    ws2, h2, eo2 = mr.forward_workspace(tables, H, D, d["x"].dtype)
    eo2.fill_(float("nan"))
    y2 = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y2,
                          workspace=ws2)
    torch.cuda.synchronize()
    n = int(tables.group_sizes.sum())
    assert not torch.isnan(eo[:n]).any()
    assert torch.equal(eo[:n].view(torch.int16), eo2[:n].view(torch.int16))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    return tables, eo, y


def _oracle(d, tokens=None):
    dt = ORACLE_DT[d["x"].dtype]
    if tokens is None:
        return oracle.moe_forward(dt, storage(d["x"]), storage(d["w_gate"]), storage(d["w_up"]),
                                  storage(d["w_down"]), d["topk_ids"].cpu().numpy(),
                                  d["topk_weights"].cpu().numpy(), want_pairs=True)
    # only the experts the tokens use
    ids = d["topk_ids"].cpu().numpy()[tokens]
    used = np.unique(ids[ids >= 0])
    remap = np.full(d["E"], -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sel = torch.from_numpy(used).long().to(DEV)
    sub_ids = np.where(ids >= 0, remap[np.maximum(ids, 0)], -1).astype(np.int32)
    return oracle.moe_forward(dt, storage(d["x"][torch.from_numpy(tokens).long().to(DEV)]),
                              storage(d["w_gate"][sel]), storage(d["w_up"][sel]),
                              storage(d["w_down"][sel]), sub_ids,
                              d["topk_weights"].cpu().numpy()[tokens], want_pairs=True)


def _check_expert_out(tables, eo, ep, K, tokens):
    """Sorted rows of expert_out against the oracle's per-slot rows."""
    pos = tables.token_topk_to_pos.cpu().numpy()
    eg = eo.float().cpu().numpy()
    got, ref = [], []
    for i, t in enumerate(tokens):
        for k in range(K):
            p = pos[t * K + k]
            if p >= 0:
                got.append(eg[p])
                ref.append(ep[i * K + k])
    if not got:
        return
    got, ref = np.stack(got), np.stack(ref)
    m = metrics(got, ref)
    assert m[1] <= 5e-3 and m[0] <= 2e-2 * max(1.0, float(np.abs(ref).max())), ("eo", m)


@pytest.mark.parametrize("ci", [0, 1])
def test_fused_small_workloads_full(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    tables, eo, y = _run_both(d, block_m=32)
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, cfg["name"])
    _check_expert_out(tables, eo, ep, cfg["K"], range(cfg["T"]))


@pytest.mark.parametrize("block_m", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_ragged(dtype, block_m):
    d = _custom(T=97, H=512, D=384, E=6, K=3, dtype=dtype, seed=11, mask=0.15, hot=2)
    tables, eo, y = _run_both(d, block_m)
    assert tables.group_sizes.cpu().numpy().max() > 2 * block_m   # an expert spans several blocks
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "ragged")
    _check_expert_out(tables, eo, ep, 3, range(97))


@pytest.mark.parametrize("H,D", [(1536, 1280), (256, 128), (512, 2048)])
def test_fused_reduction_lengths(H, D):
    """Gate/up over 24 chunks and down over 20 (full groups of steps and a
    tail at depths 6 and 8); 4 and 2 chunks (the depth-2 form); d_expert
    2048 (the whole LDS h)."""
    d = _custom(T=70, H=H, D=D, E=5, K=3, dtype="bf16", seed=16, mask=0.1, hot=1)
    tables, eo, y = _run_both(d, 32)
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "reduction lengths")
    _check_expert_out(tables, eo, ep, 3, range(70))


def test_fused_empty_experts_and_masked_tokens():
    d = _custom(T=40, H=256, D=128, E=16, K=2, dtype="bf16", seed=12)
    ids = d["topk_ids"]
    ids[ids >= 8] = 3                 # experts 8..15 get no rows
    ids[5] = -1                       # token 5 fully masked
    ids[:, 1] = torch.where(ids[:, 1] == ids[:, 0], -1, ids[:, 1])
    d["topk_ids"] = ids.contiguous()
    tables, eo, y = _run_both(d, 16)
    assert torch.all(y[5] == 0)
    y_ref, hp, ep = _oracle(d)
    assert_close_16(y.float().cpu().numpy(), y_ref, "empty experts")


def test_fused_every_slot_masked():
    mr = _mr()
    d = _custom(T=12, H=256, D=128, E=4, K=2, dtype="bf16", seed=17)
    d["topk_ids"] = torch.full_like(d["topk_ids"], -1)
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 4, block_m=32)
    y = torch.full((12, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    mr.moe_routed_forward_fused(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_fused_decode_workload_full_size():
    mr = _mr()
    cfg = S.CONFIGS[2]
    d = S.make_moe_inputs(cfg, device=DEV)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"])
    assert block_m <= 32
    tables, eo, y = _run_both(d, block_m)
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m, full_upto=0)
    y_ref, hp, ep = _oracle(d, tokens)
    assert_close_16(y.float().cpu().numpy()[tokens], y_ref, cfg["name"])
    _check_expert_out(tables, eo, ep, cfg["K"], list(tokens))
    del d, eo, y, tables
    torch.cuda.empty_cache()


def test_fused_argument_errors():
    mr = _mr()
    d = _custom(T=8, H=256, D=128, E=4, K=2, dtype="bf16", seed=15)
    big = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 4, block_m=64)
    with pytest.raises(mr.MoeError) as ei:       # row blocks larger than 32
        mr.moe_expert_fused(d["x"], d["w_gate"], d["w_up"], d["w_down"], big)
    assert ei.value.status == 4
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], 4, block_m=32)
    Dbig = mr.FUSED_MAX_D_EXPERT + 128
    wg = torch.zeros(4, Dbig, 256, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(4, 256, Dbig, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mr.MoeError) as ei:       # h of a block would not fit in LDS
        mr.moe_expert_fused(d["x"], wg, wg, wd, tables)
    assert ei.value.status == 4
    with pytest.raises(mr.MoeError) as ei:       # fp32 is the two-kernel debug path only
        mr.moe_expert_fused(d["x"].float(), d["w_gate"].float(), d["w_up"].float(),
                            d["w_down"].float(), tables)
    assert ei.value.status == 3
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(mr.MoeError) as ei:       # workspace shorter than expert_out
        mr.moe_routed_forward_fused(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables,
                                    workspace=ws)
    assert ei.value.status == 5
