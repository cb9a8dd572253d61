"""W8A8 experts on the GPU (FP8 E4M3 activations against FP8 E4M3 weights,
one fp32 scale per row of each operand) against the oracle's W8A8 forward,
which quantizes the same 16-bit inputs itself.

  * the activation quantizer (moe_quantize_fp8_rows on [rows, cols]): codes
    and scales bit for bit equal to the oracle's;
  * the FP8 MFMA path reads every E4M3 code exactly: the down GEMM with
    one-hot activation rows returns s_a * s_w * decoded code for all 254
    finite codes; with integer-valued codes and power-of-two scales every
    sum is exact in any order, so expert_out equals the exact value rounded
    to bf16, bit for bit (also through a 256-row block: the LDS-tiled pass's
    upper row half);
  * the forward against the oracle: the tiny and mid-size workloads in full
    with the per-stage intermediates, ragged shapes with masked slots and a
    hot expert at every block_m, and the decode / prefill / skewed workloads
    at full size on a token set covering every row group of every row block
    of every active expert. Tolerances as the 16-bit forward.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import ORACLE_DT, assert_close_16, cover_tokens, gpu_available, metrics, storage
from test_gpu_fp8w import _fp8_pair

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _run(d, gpu, block_m=None):
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], E, block_m=block_m)
    ws, h, eo, xq, sx, hq, sh = mr.forward_w8a8_workspace(tables, H, D, d["x"].dtype)
    h.fill_(float("nan"))
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward_w8a8(d["x"], gpu[0], gpu[1], gpu[2], tables, y=y, workspace=ws)
    torch.cuda.synchronize()
    return tables, h, eo, xq, sx, y


def _oracle(d, ref, tokens=None, want_pairs=False):
    (cg, sg), (cu, su), (cd, sd) = ref
    return oracle.moe_forward_w8a8(ORACLE_DT[d["x"].dtype], storage(d["x"]), cg, cu, cd, sg, su,
                                   sd, d["topk_ids"].cpu().numpy(),
                                   d["topk_weights"].cpu().numpy(), tokens=tokens,
                                   want_pairs=want_pairs)


def _check_x_quant(d, xq, sx):
    codes, scales = oracle.quantize_fp8_rows(ORACLE_DT[d["x"].dtype], storage(d["x"]))
    assert np.array_equal(xq.cpu().numpy(), codes)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), scales.view(np.uint32))


def _check_pairs(tables, h, eo, hp, ep):
    pos = tables.token_topk_to_pos.cpu().numpy()
    hg, eg = h.float().cpu().numpy(), eo.float().cpu().numpy()
    rows = [(pos[s], s) for s in range(pos.size) if pos[s] >= 0]
    gh = np.stack([hg[p] for p, _ in rows]); rh = np.stack([hp[s] for _, s in rows])
    ge = np.stack([eg[p] for p, _ in rows]); re = np.stack([ep[s] for _, s in rows])
    assert not np.isnan(gh).any() and not np.isnan(ge).any()
    mh, me = metrics(gh, rh), metrics(ge, re)
    assert mh[1] <= 5e-3 and mh[0] <= 2e-2 * max(1.0, float(np.abs(rh).max())), ("h", mh)
    assert me[1] <= 5e-3 and me[0] <= 2e-2 * max(1.0, float(np.abs(re).max())), ("eo", me)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
# Rows held in registers up to 8192 values (512 / 520: either side of the
# first step of that form), read twice beyond (8200).
@pytest.mark.parametrize("cols", [512, 520, 2048, 8192, 8200])
def test_activation_quantizer_bit_exact(dtype, cols):
    mr = _mr()
    g = torch.Generator().manual_seed(9 + cols)
    a = torch.randn(37, cols, generator=g)
    a[3] = 0.0
    a[5, ::3] *= 200.0
    a = a.to(dtype).to(DEV)
    q, s = mr.quantize_fp8_act_rows(a)
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_fp8_rows(ORACLE_DT[dtype], storage(a))
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), scales.view(np.uint32))


def _down_exact(hq_codes, sh, w_codes, sw, block_m, out_shift=0):
    """moe_expert_down_w8a8 on given codes / scales (E = 1, every row to
    expert 0) and the exact result, rounded to bf16. out_shift: expert_out
    starts that many elements into its allocation (2-byte steps off a
    16-byte boundary)."""
    mr = _mr()
    P, D = hq_codes.shape
    H = w_codes.shape[0]
    ids = torch.zeros(P, 1, dtype=torch.int32, device=DEV)
    tables = mr.moe_dispatch(ids, None, 1, block_m=block_m)
    w8 = mr.FP8Weights(torch.from_numpy(w_codes[None]).to(DEV), torch.from_numpy(sw[None]).to(DEV))
    buf = torch.full((P * H + out_shift,), float("nan"), dtype=torch.bfloat16, device=DEV)
    eo = buf[out_shift:].view(P, H)
    mr.moe_expert_down_w8a8(torch.from_numpy(hq_codes).to(DEV), torch.from_numpy(sh).to(DEV), w8,
                            tables, torch.bfloat16, expert_out=eo)
    torch.cuda.synchronize()
    dh = oracle.to_f32(hq_codes, oracle.FP8).astype(np.float64)
    dw = oracle.to_f32(w_codes, oracle.FP8).astype(np.float64)
    exact = (dh @ dw.T) * sh[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return eo.float().cpu().numpy(), want


def test_down_reads_every_code_exactly():
    """One-hot activation rows (code 1.0 at column i % D, scale 2^-(i%3)):
    expert_out[i, c] = s_a * s_w[c] * decode(w[c, i % D]), exact."""
    H, D = 256, 128
    P = 128
    w = (np.arange(H * D, dtype=np.int64).reshape(H, D) * 7) % 256
    w[(w == 0x7f) | (w == 0xff)] = 0                         # the two NaN codes
    w = w.astype(np.uint8)
    hq = np.zeros((P, D), np.uint8)
    hq[np.arange(P), np.arange(P) % D] = 0x38                 # E4M3 1.0
    sh = np.exp2(-(np.arange(P) % 3)).astype(np.float32)
    sw = np.exp2(-(np.arange(H) % 5)).astype(np.float32)
    got, want = _down_exact(hq, sh, w, sw, 32)
    assert np.array_equal(got, want)
    seen = np.unique(w[:, np.arange(P) % D])
    assert seen.size == 254


@pytest.mark.parametrize("block_m,P,shift", [(32, 300, 0), (256, 300, 0), (128, 300, 0),
                                             (256, 170, 0), (256, 100, 0), (256, 170, 1),
                                             (128, 300, 3)])
def test_down_exact_integer_sums(block_m, P, shift):
    """Integer-valued codes (|v| <= 8) and power-of-two scales: every partial
    sum is an exact fp32 integer, whatever the MFMA's order. The LDS-tiled
    pass cuts its tile to 64, 128, 192 or 256 rows by the block's rows: 300
    rows at block_m 256 are blocks of 256 and 44 rows, at 128 of 128, 128
    and 44; 170 and 100 rows are one block each. A shifted expert_out (not
    16-byte aligned) takes the tile epilogue's 2-byte stores."""
    rng = np.random.default_rng(4 + P)
    H, D = 256, 512
    ints = {1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4a, 6: 0x4c, 7: 0x4e, 8: 0x50}
    def codes(shape):
        v = rng.integers(1, 9, size=shape)
        c = np.vectorize(ints.get)(v).astype(np.uint8)
        return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)
    hq, w = codes((P, D)), codes((H, D))
    sh = np.exp2(-rng.integers(0, 6, size=P)).astype(np.float32)
    sw = np.exp2(-rng.integers(0, 6, size=H)).astype(np.float32)
    got, want = _down_exact(hq, sh, w, sw, block_m, out_shift=shift)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ci", [0, 1])
def test_forward_w8a8_small_workloads_full(ci):
    d = S.make_moe_inputs(S.CONFIGS[ci], device=DEV)
    gpu, ref = _fp8_pair(d)
    tables, h, eo, xq, sx, y = _run(d, gpu)
    _check_x_quant(d, xq, sx)
    y_ref, hp, ep = _oracle(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "w8a8 %s" % S.CONFIGS[ci]["name"])
    _check_pairs(tables, h, eo, hp, ep)


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
def test_forward_w8a8_ragged(block_m):
    cfg = dict(name="custom", dtype="bf16", T=300, H=512, D=384, E=5, K=3, renorm=True,
               zipf=False, seed=33)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone()
    g = torch.Generator().manual_seed(33)
    sel = (torch.rand(cfg["T"], generator=g) < 0.95).to(DEV)
    ids[:, 0] = torch.where(sel, torch.full_like(ids[:, 0], 2), ids[:, 0])   # a hot expert
    ids[:, 1:] = torch.where(ids[:, 1:] == ids[:, :1], -1, ids[:, 1:])
    ids[(torch.rand(cfg["T"], cfg["K"], generator=g) < 0.1).to(DEV)] = -1
    d["topk_ids"] = ids.contiguous()
    gpu, ref = _fp8_pair(d)
    tables, h, eo, xq, sx, y = _run(d, gpu, block_m=block_m)
    assert tables.group_sizes.max() > 256
    y_ref, hp, ep = _oracle(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "w8a8 ragged bm=%d" % block_m)
    _check_pairs(tables, h, eo, hp, ep)


def test_forward_w8a8_fp16():
    cfg = dict(S.CONFIGS[1], dtype="f16", T=128)
    d = S.make_moe_inputs(cfg, device=DEV)
    gpu, ref = _fp8_pair(d)
    tables, h, eo, xq, sx, y = _run(d, gpu)
    y_ref, hp, ep = _oracle(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "w8a8 fp16")
    _check_pairs(tables, h, eo, hp, ep)


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_forward_w8a8_full_size_sampled(ci):
    mr = _mr()
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    gpu, ref = _fp8_pair(d)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"])
    tables, h, eo, xq, sx, y = _run(d, gpu, block_m=block_m)
    _check_x_quant(d, xq, sx)
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m, full_upto=0,
                          group_rows=128)   # a covering set: the whole decode workload is 100 s of oracle time
    y_ref = _oracle(d, ref, tokens=tokens)
    got = y.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert_close_16(got[tokens], y_ref, "w8a8 %s sampled" % cfg["name"])
    del d, gpu, tables, h, eo, y
    torch.cuda.empty_cache()


def test_w8a8_argument_errors():
    mr = _mr()
    d = S.make_moe_inputs(S.CONFIGS[1], device=DEV)
    q = mr.quantize_fp8_rows(d["w_gate"])
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], d["E"])
    xq, sx = mr.quantize_fp8_act_rows(d["x"])
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_expert_gate_up_w8a8(xq, sx, d["w_gate"], d["w_up"], tables)
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_expert_gate_up_w8a8(xq, sx, q, q, tables, dtype=torch.float32)
    with pytest.raises(mr.MoeError, match="MOE_ERR_SHAPE"):
        mr.moe_expert_gate_up_w8a8(xq[:-1], sx[:-1], q, q, tables)
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_routed_forward_w8a8(d["x"].float(), q, q, q, tables)
