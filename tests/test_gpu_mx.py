"""Block-scaled (MX) experts on the GPU against the oracle (same seeded inputs).

  * the MX quantizer (moe_quantize_mx_rows): MXFP8 and MXFP4 codes and E8M0
    scales bit for bit equal to the oracle's, for bf16 / fp16 / fp32 inputs
    with zero blocks, tiny blocks, outliers and the E2M1 tie cases;
  * the grouped MX down GEMM on inputs whose every product and partial sum
    is exact in fp32 (so the MFMA's summation order cannot matter): each
    32-block has its own scale on both operands, so a scale applied to the
    wrong block, a misordered FP4 nibble or a transposed operand changes the
    bf16 result -- compared bit for bit against the exact sum;
  * the MX forward against the oracle's MX forward: the quantised x bit for
    bit, h / expert_out per routed pair and y at the graded tolerance, at
    the mid-size workload, ragged shapes at every block_m, fp16, and sampled
    tokens of the DeepSeek decode / prefill / skewed workloads.
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


def _rows_input(dtype, rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(rows, cols, generator=g)
    a[0, :64] = 0.0                                         # zero blocks
    a[1] *= 1e-6                                            # tiny blocks
    a[2, ::7] *= 300.0                                      # outliers
    ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, -0.25, -5.0, 4.0])
    a[3, :12] = ties
    a[3, 12:32] = 0.5                                       # block max 7 -> X = 1 for FP4
    return a.to(dtype).to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("fmt", [0, 4])
def test_quantize_mx_rows_bit_exact(dtype, fmt):
    mr = _mr()
    a = _rows_input(dtype, 37, 2048, 3)
    c, s = mr.quantize_mx_rows(a, fmt)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mx_rows(ORACLE_DT[dtype], storage(a), fmt)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(c.cpu().numpy(), rc)


def _grid4():
    return np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _exact_rows(rng, rows, cols, fmt):
    """Rows whose 32-blocks are exactly representable with a random scale
    per block: MXFP4 -- E2M1 values with a 6 in each block; MXFP8 -- small
    integers with a 448 in each block (a multiple of 0.5 with at most 4
    significant bits)."""
    if fmt == 4:
        g = _grid4()
        v = rng.choice(np.concatenate([-g, g]), size=(rows, cols))
        v[:, ::32] = 6.0
    else:
        v = rng.integers(-16, 17, size=(rows, cols)).astype(np.float64) / 2
        v[:, ::32] = 448.0
    # scales 2^-1 .. 2^1: every product is a multiple of 2^-4 and every
    # partial sum of a 512-long row stays below 2^20, exact in fp32
    k = rng.integers(-1, 2, size=(rows, cols // 32))
    return (v * 2.0 ** np.repeat(k, 32, axis=1)).astype(np.float32)


def _shifted(a, shift):
    """Device copy of uint8 array a whose data starts `shift` bytes past an
    aligned allocation (shift 0: a plain copy)."""
    buf = torch.empty(a.size + shift, dtype=torch.uint8, device=DEV)
    v = buf[shift:].view(a.shape)
    v.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return v


def _down_case(T, H, D, E, K, block_m, seed, scale_shift=0):
    mr = _mr()
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[:, 0] = np.where(np.arange(T) % 3 == 0, 1, ids[:, 0])
    ids[:, 1:] = np.where(ids[:, 1:] == ids[:, :1], -1, ids[:, 1:])
    ids[::7, -1] = -1
    w = rng.uniform(0.1, 1, size=(T, K)).astype(np.float32)
    P = T * K
    hv = _exact_rows(rng, P, D, 0)
    hc, hs = oracle.quantize_mx_rows(oracle.F32, hv, 0)
    assert np.array_equal(oracle.mx_decode(hc, hs, 0), hv)
    wv = _exact_rows(rng, E * H, D, 4)
    wc, ws = oracle.quantize_mx_rows(oracle.F32, wv, 4)
    assert np.array_equal(oracle.mx_decode(wc, ws, 4), wv)
    tables = mr.moe_dispatch(torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), E,
                             block_m=block_m)
    wmx = mr.MXWeights(torch.from_numpy(wc.reshape(E, H, D // 2)).to(DEV),
                       _shifted(ws.reshape(E, H, D // 32), scale_shift))
    eo = torch.full((P, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    mr.moe_expert_down_mx(torch.from_numpy(hc).to(DEV), _shifted(hs, scale_shift), wmx, tables,
                          torch.bfloat16, expert_out=eo)
    torch.cuda.synchronize()
    sizes = tables.group_sizes.cpu().numpy()
    offs = tables.group_offsets.cpu().numpy()
    got = eo.float().cpu().numpy()
    assert not np.isnan(got[:int(sizes.sum())]).any()
    wv3 = wv.reshape(E, H, D).astype(np.float64)
    for e in range(E):
        if sizes[e] == 0:
            continue
        rows = slice(offs[e], offs[e] + sizes[e])
        exact = hv[rows].astype(np.float64) @ wv3[e].T            # exact in float64 and fp32
        want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
        assert np.array_equal(got[rows], want), "expert %d" % e


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
def test_down_mx_exact(block_m):
    _down_case(T=200, H=512, D=512, E=5, K=3, block_m=block_m, seed=block_m + 1)


# Reduction lengths of an odd (768) and an even (1024) number of 256-long
# chunks, and scale arrays 4 bytes off a 16-byte boundary: the down GEMM
# loads two chunks' scale words at once only for an even chunk count and
# 16-byte aligned scales, and takes the per-chunk loads otherwise.
@pytest.mark.parametrize("D,block_m,shift", [(768, 16, 0), (1024, 32, 0), (1024, 16, 4),
                                             (1024, 64, 4)])
def test_down_mx_exact_scale_loads(D, block_m, shift):
    _down_case(T=120, H=256, D=D, E=4, K=2, block_m=block_m, seed=D + block_m + shift,
               scale_shift=shift)


def _mx_weights(d):
    mr = _mr()
    gpu, ref = [], []
    for n in ("w_gate", "w_up", "w_down"):
        q = mr.quantize_mx_weights(d[n])
        torch.cuda.synchronize()
        rc, rs = oracle.quantize_mx_rows(ORACLE_DT[d[n].dtype], storage(d[n]), 4)
        assert np.array_equal(q.packed.cpu().numpy(), rc), n
        assert np.array_equal(q.scales.cpu().numpy(), rs), n
        gpu.append(q)
        ref.append((rc, rs))
    return gpu, ref


def _run_mx(d, gpu, block_m=None):
    mr = _mr()
    T, H, D, E = d["T"], d["H"], d["D"], d["E"]
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], E, block_m=block_m)
    ws, h, eo, xq, xs, hq, hs = mr.forward_mx_workspace(tables, H, D, d["x"].dtype)
    h.fill_(float("nan"))
    eo.fill_(float("nan"))
    y = torch.full((T, H), float("nan"), dtype=d["x"].dtype, device=DEV)
    mr.moe_routed_forward_mx(d["x"], gpu[0], gpu[1], gpu[2], tables, y=y, workspace=ws)
    torch.cuda.synchronize()
    return tables, h, eo, xq, xs, y


def _oracle_mx(d, ref, tokens=None, want_pairs=False):
    (cg, sg), (cu, su), (cd, sd) = ref
    return oracle.moe_forward_mx(ORACLE_DT[d["x"].dtype], storage(d["x"]), cg, cu, cd, sg, su, sd,
                                 d["topk_ids"].cpu().numpy(), d["topk_weights"].cpu().numpy(),
                                 tokens=tokens, want_pairs=want_pairs)


def _check_x_quant(d, xq, xs):
    rc, rs = oracle.quantize_mx_rows(ORACLE_DT[d["x"].dtype], storage(d["x"]), 0)
    assert np.array_equal(xq.cpu().numpy(), rc)
    assert np.array_equal(xs.cpu().numpy(), rs)


def _check_pairs(tables, h, eo, hp, ep):
    pos = tables.token_topk_to_pos.cpu().numpy()
    hg, eg = h.float().cpu().numpy(), eo.float().cpu().numpy()
    rows = [(pos[s], s) for s in range(pos.size) if pos[s] >= 0]
    gh = np.stack([hg[p] for p, _ in rows]); rh = np.stack([hp[s] for _, s in rows])
    ge = np.stack([eg[p] for p, _ in rows]); re = np.stack([ep[s] for _, s in rows])
    assert not np.isnan(gh).any() and not np.isnan(ge).any()
    mh, me = metrics(gh, rh), metrics(ge, re)
    assert mh[1] <= 5e-3 and mh[0] <= 2e-2 * max(1.0, float(np.abs(rh).max())), ("h", mh)
    assert me[1] <= 1e-2 and me[0] <= 4e-2 * max(1.0, float(np.abs(re).max())), ("eo", me)


def test_forward_mx_mid_full():
    d = S.make_moe_inputs(S.CONFIGS[1], device=DEV)
    gpu, ref = _mx_weights(d)
    tables, h, eo, xq, xs, y = _run_mx(d, gpu)
    _check_x_quant(d, xq, xs)
    y_ref, hp, ep = _oracle_mx(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "mx %s" % S.CONFIGS[1]["name"])
    _check_pairs(tables, h, eo, hp, ep)


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
def test_forward_mx_ragged(block_m):
    cfg = dict(name="custom", dtype="bf16", T=300, H=512, D=512, E=5, K=3, renorm=True,
               zipf=False, seed=51)
    d = S.make_moe_inputs(cfg, device=DEV)
    ids = d["topk_ids"].clone()
    ids[torch.arange(0, 300, 7, device=DEV), 1] = -1
    ids[:, 0] = torch.where(torch.arange(300, device=DEV) % 3 == 0, 2, ids[:, 0])
    ids[:, 1:] = torch.where(ids[:, 1:] == ids[:, :1], -1, ids[:, 1:])
    d["topk_ids"] = ids.contiguous()
    gpu, ref = _mx_weights(d)
    tables, h, eo, xq, xs, y = _run_mx(d, gpu, block_m=block_m)
    y_ref, hp, ep = _oracle_mx(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "mx ragged bm=%d" % block_m)
    _check_pairs(tables, h, eo, hp, ep)


def test_forward_mx_fp16():
    cfg = dict(name="custom-f16", dtype="f16", T=96, H=256, D=256, E=4, K=2, renorm=False,
               zipf=False, seed=53)
    d = S.make_moe_inputs(cfg, device=DEV)
    gpu, ref = _mx_weights(d)
    tables, h, eo, xq, xs, y = _run_mx(d, gpu)
    _check_x_quant(d, xq, xs)
    y_ref, hp, ep = _oracle_mx(d, ref, want_pairs=True)
    assert_close_16(y.float().cpu().numpy(), y_ref, "mx fp16")
    _check_pairs(tables, h, eo, hp, ep)


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_forward_mx_full_size_sampled(ci):
    mr = _mr()
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, device=DEV)
    gpu, ref = _mx_weights(d)
    block_m = mr.default_block_m(cfg["T"], cfg["K"], cfg["E"], "mx")   # as the benchmark
    tables, h, eo, xq, xs, y = _run_mx(d, gpu, block_m=block_m)
    _check_x_quant(d, xq, xs)
    # one checked row in every scheduled row block (the MX oracle decodes
    # every weight block per dot product: the slowest of the oracles)
    tokens = cover_tokens(d["topk_ids"].cpu().numpy(), cfg["E"], block_m, full_upto=0,
                          group_rows=256)
    y_ref = _oracle_mx(d, ref, tokens=tokens)
    got = y.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert_close_16(got[tokens], y_ref, "mx %s sampled" % cfg["name"])


def test_mx_argument_errors():
    mr = _mr()
    d = S.make_moe_inputs(S.CONFIGS[1], device=DEV)
    q = mr.quantize_mx_weights(d["w_gate"])
    tables = mr.moe_dispatch(d["topk_ids"], d["topk_weights"], d["E"])
    xq, xs = mr.quantize_mx_rows(d["x"], mr.MX_FP8)
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.moe_expert_gate_up_mx(xq, xs, d["w_gate"], d["w_up"], tables)
    with pytest.raises(mr.MoeError, match="MOE_ERR_SHAPE"):
        mr.MXWeights(q.packed, q.scales[:, :, :-1].contiguous())
    with pytest.raises(mr.MoeError, match="MOE_ERR_SHAPE"):
        mr.quantize_mx_rows(d["x"][:, :100].contiguous())
    with pytest.raises(mr.MoeError, match="MOE_ERR_DTYPE"):
        mr.quantize_mx_rows(d["x"], fmt=3)
