"""moe_reduce_fused on the GPU against the oracle (same seeded inputs).

Cases follow the TileOPs-Metax moe_reduce_fused PR's correctness list (shapes
T x K x H, fp16/bf16/fp32, no-weights path, -1 skip, error cases) plus the
skewed workload's standalone reduce at full size. Both sides accumulate with
fused multiply-adds in k order, so the fp32 sums are expected bit-identical;
the graded bar is the tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import ORACLE_DT, assert_close_16, gpu_available, metrics, storage

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _inputs(T, K, H, dtype, seed, mask=0.1, R=None):
    d = S.make_reduce_inputs(T, K, H, dtype=dtype, seed=seed, mask_frac=mask, device=DEV, R=R)
    return d["expert_out"], d["token_topk_to_pos"], d["topk_weights"]


def _check(x, pos, w, out_dtype):
    mr = _mr()
    y = torch.full((pos.shape[0], x.shape[1]), float("nan"), dtype=out_dtype, device=DEV)
    mr.moe_reduce_fused(x, pos, w, out_dtype=out_dtype, y=y)
    torch.cuda.synchronize()
    ref = oracle.reduce(ORACLE_DT[x.dtype], storage(x), pos.cpu().numpy(),
                        None if w is None else w.cpu().numpy())
    got = y.float().cpu().numpy()
    if out_dtype == torch.float32:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), metrics(got, ref)
    else:
        exp = torch.from_numpy(ref).to(out_dtype).float().numpy()
        assert_close_16(got, ref, "reduce")
        assert np.array_equal(got, exp), "not bit-identical to the k-ordered fma sum"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("T,K,H", [(4, 2, 256), (16, 2, 512), (32, 8, 3072), (32, 8, 7168),
                                   (512, 8, 7168), (1, 8, 256), (8, 1, 256), (33, 3, 768)])
def test_reduce_shapes(T, K, H, dtype):
    x, pos, w = _inputs(T, K, H, dtype, seed=T + K + H)
    _check(x, pos, w, x.dtype)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_reduce_out_dtype(out_dtype):
    x, pos, w = _inputs(64, 8, 1024, "bf16", seed=5)
    _check(x, pos, w, out_dtype)


def test_reduce_without_weights():
    x, pos, _ = _inputs(48, 4, 512, "bf16", seed=6)
    _check(x, pos, None, torch.bfloat16)


def test_reduce_skips_masked_and_never_reads_them():
    mr = _mr()
    T, K, H = 6, 4, 256
    x = torch.randn(T * K + 1, H, device=DEV).to(torch.bfloat16)
    x[-1] = float("nan")                    # the row a wrapped -1 would read
    pos = torch.arange(T * K, device=DEV, dtype=torch.int32).view(T, K).contiguous()
    pos[1] = -1                              # token 1: all slots masked
    pos[3, ::2] = -1
    w = torch.rand(T, K, device=DEV)
    y = mr.moe_reduce_fused(x, pos, w)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.all(y[1] == 0)
    _check(x, pos, w, torch.bfloat16)


def test_reduce_out_of_range_positions_are_skipped():
    mr = _mr()
    x = torch.ones(8, 256, device=DEV, dtype=torch.bfloat16)
    pos = torch.tensor([[0, 8], [1, 7]], device=DEV, dtype=torch.int32)
    y = mr.moe_reduce_fused(x, pos, None, out_dtype=torch.float32)
    assert y.cpu().tolist() == [[1.0] * 256, [2.0] * 256]


def test_reduce_skewed_workload_full_size():
    cfg = S.CONFIGS[4]
    x, pos, w = _inputs(cfg["T"], cfg["K"], cfg["H"], "bf16", seed=cfg["seed"])
    assert int((pos == -1).sum()) == int(0.1 * cfg["T"] * cfg["K"])
    _check(x, pos, w, torch.bfloat16)


def test_reduce_error_cases():
    mr = _mr()
    x, pos, w = _inputs(4, 2, 256, "bf16", seed=1)
    with pytest.raises(mr.MoeError) as ei:                      # H % 256 != 0
        mr.moe_reduce_fused(torch.zeros(8, 320, device=DEV, dtype=torch.bfloat16), pos, w)
    assert ei.value.status == 2
    with pytest.raises(mr.MoeError) as ei:                      # weights dtype
        mr.moe_reduce_fused(x, pos, w.half())
    assert ei.value.status == 3
    with pytest.raises(mr.MoeError) as ei:                      # shape mismatch
        mr.moe_reduce_fused(x, pos, w[:, :1].contiguous())
    assert ei.value.status == 2
