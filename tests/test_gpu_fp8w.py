"""FP8 expert weights on the GPU against the oracle (same seeded inputs).

  * the quantizer (moe_quantize_fp8_rows): codes and scales bit for bit equal
    to the oracle's, for bf16 / fp16 / fp32 weights, zero rows and wide
    dynamic ranges, and on the full DeepSeek-shaped weights;
  * the FP8 grouped GEMMs read every E4M3 code exactly: the down GEMM with
    one-hot h rows returns scale x decoded code for all 254 finite codes;
  * the forward with FP8 weights against the oracle's FP8 forward (which
    quantizes the same 16-bit weights itself): the tiny and mid-size
    workloads in full with the per-stage intermediates, ragged shapes at
    every block_m, and the decode / prefill / skewed workloads at full size
    on sampled tokens. Tolerances as the 16-bit forward.
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


def _quant_pair(w):
    """GPU quantizer output and the oracle's, for a stacked weight tensor."""
    q = _mr().quantize_fp8_rows(w)
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_fp8_rows(ORACLE_DT[w.dtype], storage(w))
    return q, codes, scales


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_quantizer_bit_exact(dtype):
    g = torch.Generator().manual_seed(5)
    w = torch.randn(3, 40, 320, generator=g)
    w[0, 3] = 0.0                                            # zero row
    w[1, 7] *= 1e-4                                          # tiny row
    w[2, 9, ::7] *= 300.0                                    # outliers
    w = w.to(dtype).to(DEV)
    q, codes, scales = _quant_pair(w)
    assert np.array_equal(q.codes.cpu().numpy(), codes)
    assert np.array_equal(q.scales.cpu().numpy().view(np.uint32), scales.view(np.uint32))


def test_down_gemm_reads_every_code_exactly():
    """expert_out[i, c] = R(s[c] * sum_j h[i, j] * q[c, j]) with one-hot h rows
    and power-of-two scales is exactly s[c] * decode(q[c, j]) in bf16."""
    mr = _mr()
    H, D, E, K = 256, 128, 1, 1
    T = 128                                                  # one h row per column j
    ids = torch.zeros(T, K, dtype=torch.int32, device=DEV)
    tables = mr.moe_dispatch(ids, None, E, block_m=32)
    codes = np.arange(H * D, dtype=np.int64).reshape(H, D) % 256
    codes[(codes == 0x7f) | (codes == 0xff)] = 0             # the two NaN codes
    codes = codes.astype(np.uint8)[None]
    scales = np.exp2(-(np.arange(H) % 5)).astype(np.float32)[None]
    w8 = mr.FP8Weights(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    h = torch.zeros(T, D, dtype=torch.bfloat16, device=DEV)
    h[torch.arange(T), torch.arange(T) % D] = 1.0            # sorted row i = token i (stable)
    eo = mr.moe_expert_down_w8(h, w8, tables)
    torch.cuda.synchronize()
    dec = oracle.to_f32(codes[0], oracle.FP8)                # [H, D]
    want = (dec * scales[0][:, None]).T[np.arange(T) % D]    # [T, H]
    got = eo.float().cpu().numpy()
    assert np.array_equal(got, want)


def _fp8_pair(d):
    """GPU-quantized weights (checked bit-exact against the oracle's) and the
    oracle's codes / scales for its own forward."""
    gpu, ref = [], []
    for n in ("w_gate", "w_up", "w_down"):
        q, c, s = _quant_pair(d[n])
        assert np.array_equal(q.codes.cpu().numpy(), c), n
        assert np.array_equal(q.scales.cpu().numpy().view(np.uint32), s.view(np.uint32)), n
        gpu.append(q)
        ref.append((c, s))
    return gpu, ref


def _run_w8(d, gpu, block_m=None):
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], E, block_m=block_m)
    ws, h, eo = mr.forward_workspace(tables, H, D, d["x"].dtype)
    h.fill_(float("nan"))
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward_w8(d["x"], gpu[0], gpu[1], gpu[2], tables, y=y, workspace=ws)
    torch.cuda.synchronize()
    return tables, h, eo, y


def _oracle_w8(d, ref, tokens=None, want_pairs=False):
    (cg, sg), (cu, su), (cd, sd) = ref
    return oracle.moe_forward_w8(ORACLE_DT[d["x"].dtype], storage(d["x"]), cg, cu, cd, sg, su, sd,
                                 d["topk_ids"].cpu().numpy(), d["topk_weights"].cpu().numpy(),
                                 tokens=tokens, want_pairs=want_pairs)


def _check_pairs(tables, h, eo, hp, ep, K):
    pos = tables.token_topk_to_pos.cpu().numpy()
    hg, eg = h.float().cpu().numpy(), eo.float().cpu().numpy()
    rows = [(pos[s], s) for s in range(pos.size) if pos[s] >= 0]
    gh = np.stack([hg[p] for p, _ in rows]); rh = np.stack([hp[s] for _, s in rows])
    ge = np.stack([eg[p] for p, _ in rows]); re = np.stack([ep[s] for _, s in rows])
    assert not np.isnan(gh).any() and not np.isnan(ge).any()
    mh, me = metrics(gh, rh), metrics(ge, re)
    assert mh[1] <= 5e-3 and mh[0] <= 2e-2 * max(1.0, float(np.abs(rh).max())), ("h", mh)
    assert me[1] <= 5e-3 and me[0] <= 2e-2 * max(1.0, float(np.abs(re).max())), ("eo", me)


@pytest.mark.parametrize("ci", [0, 1])
def test_forward_w8_small_workloads_full(ci):
    d = S.make_moe_inputs(S.CONFIGS[ci], device=DEV)
    gpu, ref = _fp8_pair(d)
    tables, h, eo, y = _run_w8(d, gpu)
    y_ref, hp, ep = _oracle_w8(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "fp8 weights %s" % S.CONFIGS[ci]["name"])
    _check_pairs(tables, h, eo, hp, ep, d["K"])


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
def test_forward_w8_ragged(block_m):
    cfg = dict(name="custom", dtype="bf16", T=300, H=512, D=384, E=5, K=3, renorm=True,
               zipf=False, seed=31)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone()
    ids[torch.arange(0, 300, 7, device=DEV), 1] = -1         # masked slots
    ids[:, 0] = torch.where(torch.arange(300, device=DEV) % 3 == 0, 2, ids[:, 0])
    ids[:, 1:] = torch.where(ids[:, 1:] == ids[:, :1], -1, ids[:, 1:])
    d["topk_ids"] = ids.contiguous()
    gpu, ref = _fp8_pair(d)
    tables, h, eo, y = _run_w8(d, gpu, block_m=block_m)
    y_ref, hp, ep = _oracle_w8(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "fp8 ragged bm=%d" % block_m)
    _check_pairs(tables, h, eo, hp, ep, d["K"])


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_forward_w8_full_size_sampled(ci):
    mr = _mr()
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    gpu, ref = _fp8_pair(d)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"])
    tables, h, eo, y = _run_w8(d, gpu, block_m=block_m)
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m, full_upto=0,
                          group_rows=128)   # a covering set: the whole decode workload is 100 s of oracle time
    y_ref = _oracle_w8(d, ref, tokens=tokens)
    got = y.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert_close_16(got[tokens], y_ref, "fp8 weights %s sampled" % cfg["name"])


def test_w8_argument_errors():
    mr = _mr()
    d = S.make_moe_inputs(S.CONFIGS[0], device=DEV)
    q = mr.quantize_fp8_rows(d["w_gate"])
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], d["E"])
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_expert_gate_up_w8(d["x"], d["w_gate"], d["w_up"], tables)
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_expert_gate_up_w8(d["x"].float(), q, q, tables)
    with pytest.raises(mr.MoeError, match="MOE_ERR_SHAPE"):
        mr.FP8Weights(q.codes, q.scales[:, :-1].contiguous())
