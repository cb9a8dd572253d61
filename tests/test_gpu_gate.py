"""The router gate on the GPU against the oracle (same seeded inputs).

Logits are one fp32 fused-multiply-add chain over h ascending on both sides,
so logits and the ids decided from them must match bit for bit; the softmax
weights use tree-reduced sums on the GPU and sequential ones in the oracle,
so they agree to a few ulp (rtol 1e-5). Covered: every workload's shape at
full size (the skewed one with its Zipf logit bias), ragged sizes (T, E not
multiples of the 16 x 32 tile, E above and below 64), duplicated router rows
(ties to the lower index), K = E, and the gate feeding dispatch and the
forward end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import ORACLE_DT, assert_close_16, gpu_available, storage

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _check(x, wr, K, renorm, bias=None):
    mr = _mr()
    ids, w, logits = mr.moe_gate(x, wr, K, renorm=renorm, bias=bias)
    torch.cuda.synchronize()
    ref = oracle.gate(ORACLE_DT[x.dtype], storage(x), wr.cpu().numpy(), K, renorm,
                      bias=None if bias is None else bias.cpu().numpy())
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.allclose(w.cpu().numpy(), ref["weights"], rtol=1e-5, atol=1e-9)
    return ids, w, logits


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_gate_workloads_full_size(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV, weights=False)
    bias = S.zipf_bias(cfg["E"]).to(DEV) if cfg.get("zipf") else None
    ids, w, _ = _check(d["x"], d["router"], cfg["K"], cfg["renorm"], bias)
    # the workload recipe's router ranks float64 logits: the ids agree except
    # at near-ties (checked against the oracle's pins on the CPU)
    same = (ids.cpu() == d["topk_ids"].cpu()).all(dim=1).float().mean().item()
    assert same > 0.99


@pytest.mark.parametrize("T,H,E,K,dtype", [(37, 192, 10, 3, torch.bfloat16),
                                           (50, 128, 64, 8, torch.float16),
                                           (33, 256, 65, 2, torch.float32),
                                           (17, 64, 300, 64, torch.bfloat16),
                                           (5, 128, 1024, 7, torch.bfloat16),
                                           (3, 64, 6, 6, torch.float32)])
@pytest.mark.parametrize("renorm", [False, True])
def test_gate_ragged(T, H, E, K, dtype, renorm):
    g = torch.Generator().manual_seed(T * 1000 + E)
    x = torch.randn(T, H, generator=g).to(dtype).to(DEV)
    wr = (torch.randn(E, H, generator=g) * 0.05).to(DEV)
    _check(x, wr, K, renorm)


def test_gate_ties_to_lower_index():
    T, H, E = 9, 64, 12
    x = torch.ones(T, H, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(E, H, device=DEV)
    wr[3] = 0.25
    wr[7] = 0.25
    wr[10] = 0.125
    wr[2] = 0.125
    ids, w, _ = _check(x, wr, 4, False)
    assert (ids.cpu() == torch.tensor([3, 7, 2, 10], dtype=torch.int32)).all()


def test_gate_then_forward_end_to_end():
    """x -> moe_gate -> moe_dispatch -> moe_routed_forward on the device,
    against the oracle's gate feeding the oracle's forward."""
    mr = _mr()
    cfg = dict(S.CONFIGS[1])
    d = S.make_moe_inputs(cfg, device=DEV)
    ids, w, _ = mr.moe_gate(d["x"], d["router"], cfg["K"], renorm=cfg["renorm"])
    tables = mr.moe_dispatch(ids, w, cfg["E"])
    y = mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables)
    torch.cuda.synchronize()
    dt = ORACLE_DT[d["x"].dtype]
    g = oracle.gate(dt, storage(d["x"]), d["router"].cpu().numpy(), cfg["K"], cfg["renorm"])
    assert np.array_equal(ids.cpu().numpy(), g["ids"])
    y_ref = oracle.moe_forward(dt, storage(d["x"]), storage(d["w_gate"]), storage(d["w_up"]),
                               storage(d["w_down"]), g["ids"], g["weights"])
    assert_close_16(y.float().cpu().numpy(), y_ref, "gate + forward")


def test_gate_argument_errors():
    mr = _mr()
    x = torch.zeros(4, 96, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(8, 96, device=DEV)
    with pytest.raises(mr.MoeError, match="MOE_ERR_SHAPE"):
        mr.moe_gate(x, wr, 2)
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_gate(x[:, :64].contiguous(), wr[:, :64].contiguous().double(), 2)
