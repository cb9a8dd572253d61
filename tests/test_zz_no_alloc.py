"""moe_routed_forward_noalloc -- the forward whose workspace is the
library's static per-GPU scratch array (for callers that cannot allocate) --
against moe_routed_forward with a caller workspace, through the C ABI.

Both run the same kernels on the same tables, so the outputs must be equal
bit for bit. Three calls in a row with shrinking inputs (the DeepSeek-shaped
decode layer, whose 72 MiB workspace nearly fills the 80 MiB scratch, then
the mid-size layer, then a small ragged one) check that a call is not
affected by what an earlier, larger call left in the scratch; a call whose
workspace would not fit is rejected before anything is launched.
"""
import pytest
import torch

import synthetic as S
from helpers import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _both(d, block_m=None):
    mr = _mr()
    T, H = d["T"], d["H"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], d["E"], block_m=block_m)
    y_ref = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y=y_ref)
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward_noalloc(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y)
    torch.cuda.synchronize()
    return y_ref, y


def _ragged():
    cfg = dict(name="ragged", dtype="bf16", T=97, H=512, D=384, E=6, K=3, renorm=True,
               zipf=False, seed=11)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone()
    ids[3] = -1
    ids[10, 1] = -1
    d["topk_ids"] = ids.contiguous()
    return d


def test_noalloc_equals_forward_on_shrinking_calls():
    mr = _mr()
    cfg = S.CONFIGS[2]
    need = mr._lib.lib().moe_forward_workspace_bytes(cfg["T"], cfg["K"], cfg["H"], cfg["D"],
                                                     mr._lib.MOE_BF16)
    assert 0 < need <= mr.NOALLOC_SCRATCH_BYTES
    for i, make in enumerate((lambda: S.make_moe_inputs(S.CONFIGS[2], device=DEV),
                              lambda: S.make_moe_inputs(S.CONFIGS[1], device=DEV),
                              _ragged)):
        d = make()
        print("noalloc call %d: T=%d H=%d D=%d E=%d K=%d" % (i, d["T"], d["H"], d["D"], d["E"],
                                                            d["K"]), flush=True)
        y_ref, y = _both(d)
        assert not torch.isnan(y_ref).any()
        assert torch.equal(y, y_ref), "call %d differs" % i
        del d, y_ref, y
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    mr = _mr()
    cfg = dict(name="too-big", dtype="bf16", T=4096, H=1024, D=512, E=8, K=8, renorm=True,
               zipf=False, seed=5)
    d = S.make_moe_inputs(cfg, device=DEV)
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], d["E"])
    y = torch.full((cfg["T"], cfg["H"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mr.MoeError) as ei:
        mr.moe_routed_forward_noalloc(d["x"], d["w_gate"], d["w_up"], d["w_down"], tables, y)
    assert ei.value.status == mr._lib.MOE_ERR_WORKSPACE
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()          # nothing was launched
