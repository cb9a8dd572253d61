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
from helpers import ORACLE_DT, REL_L2_16, assert_close_16, gpu_available, metrics, storage

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


# ------------------------------------------------- scaled / FP8 variants ---
# (PR section 1: x_sf per expanded row, sf per token, FP8 E4M3 rows in / out.)
# Both sides take the same fp32 steps (w * x_sf, k-ordered fma, * sf, one
# cast), so the stored bits are compared exactly; FP8 outputs are in addition
# held to the format's rounding bound (half a unit in the last place: 2^-4
# relative for normal values, 2^-10 absolute below 2^-6).

def _fp8_rows(R, H, seed):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(R, H, generator=g) * 4.0
    return v.to(torch.float8_e4m3fn).to(DEV)


def _check_scaled(x, pos, w, x_sf, sf, out_dtype):
    mr = _mr()
    T, H = pos.shape[0], x.shape[1]
    y = torch.zeros(T, H, dtype=out_dtype, device=DEV)
    if out_dtype != torch.float8_e4m3fn:
        y.fill_(float("nan"))
    mr.moe_reduce_fused(x, pos, w, out_dtype=out_dtype, y=y, x_sf=x_sf, sf=sf)
    torch.cuda.synchronize()
    ref = oracle.reduce(ORACLE_DT[x.dtype], storage(x), pos.cpu().numpy(),
                        None if w is None else w.cpu().numpy(),
                        x_sf=None if x_sf is None else x_sf.cpu().numpy(),
                        sf=None if sf is None else sf.cpu().numpy())
    got_bits = storage(y)
    exp_bits = oracle.from_f32(ref, ORACLE_DT[out_dtype])
    assert np.array_equal(np.asarray(got_bits).view(np.uint8), np.asarray(exp_bits).view(np.uint8))
    got = y.float().cpu().numpy()
    if out_dtype == torch.float8_e4m3fn:
        lim = np.maximum(np.abs(ref) * 2.0 ** -4, 2.0 ** -10)
        inside = np.abs(ref) < 448
        assert np.all(np.abs(got - ref)[inside] <= lim[inside])
    elif out_dtype != torch.float32:
        # a single rounding to 16 bits: within half an ulp (2^-8 relative for
        # bfloat16, 2^-11 for binary16) of the fp32 sum
        half_ulp = 2.0 ** -8 if out_dtype == torch.bfloat16 else 2.0 ** -11
        assert np.all(np.abs(got - ref) <= np.abs(ref) * half_ulp + 2.0 ** -24)
        assert metrics(got, ref)[1] <= REL_L2_16
    return ref


@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32", "fp8"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32, torch.float8_e4m3fn])
@pytest.mark.parametrize("T,K,H", [(33, 3, 768), (64, 8, 7168)])
def test_reduce_scaled(in_dtype, out_dtype, T, K, H):
    seed = T + H + len(in_dtype)
    if in_dtype == "fp8":
        _, pos, w = _inputs(T, K, H, "bf16", seed=seed)
        x = _fp8_rows(T * K, H, seed)
    else:
        x, pos, w = _inputs(T, K, H, in_dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    x_sf = (torch.rand(x.shape[0], generator=g) * 1.5 + 0.25).to(DEV)
    sf = (torch.rand(T, generator=g) * 0.5 + 0.1).to(DEV)
    _check_scaled(x, pos, w, x_sf, sf, out_dtype)


@pytest.mark.parametrize("which", ["x_sf", "sf"])
def test_reduce_one_scale_only(which):
    x, pos, w = _inputs(40, 4, 1024, "bf16", seed=17)
    g = torch.Generator().manual_seed(18)
    x_sf = (torch.rand(x.shape[0], generator=g) + 0.5).to(DEV) if which == "x_sf" else None
    sf = (torch.rand(40, generator=g) + 0.5).to(DEV) if which == "sf" else None
    _check_scaled(x, pos, None, x_sf, sf, torch.float32)


def test_reduce_fp8_output_saturates():
    mr = _mr()
    x = torch.full((4, 256), 300.0, device=DEV, dtype=torch.bfloat16)
    pos = torch.tensor([[0, 1], [2, -1]], device=DEV, dtype=torch.int32)
    y = mr.moe_reduce_fused(x, pos, None, out_dtype=torch.float8_e4m3fn)
    torch.cuda.synchronize()
    b = y.view(torch.uint8).cpu()
    assert torch.all(b[0] == 0x7e)                      # 600 -> 448
    assert torch.all(b[1] == 0x79)                      # 300 -> 288 (nearest code)


def test_reduce_skewed_workload_fp8_quantized_form():
    # The quantized form at the skewed workload's full size: FP8 rows with a
    # per-row scale in, FP8 out with a per-token scale.
    cfg = S.CONFIGS[4]
    T, K, H = cfg["T"], cfg["K"], cfg["H"]
    _, pos, w = _inputs(T, K, H, "bf16", seed=cfg["seed"])
    x = _fp8_rows(T * K, H, cfg["seed"])
    g = torch.Generator().manual_seed(cfg["seed"] + 1)
    x_sf = (torch.rand(T * K, generator=g) * 0.05 + 0.01).to(DEV)
    sf = (torch.rand(T, generator=g) * 4 + 1).to(DEV)
    _check_scaled(x, pos, w, x_sf, sf, torch.float8_e4m3fn)


def test_reduce_scaled_error_cases():
    mr = _mr()
    x, pos, w = _inputs(4, 2, 256, "bf16", seed=1)
    with pytest.raises(mr.MoeError) as ei:                      # x_sf of the wrong length
        mr.moe_reduce_fused(x, pos, w, x_sf=torch.ones(3, device=DEV))
    assert ei.value.status == 2
    with pytest.raises(mr.MoeError) as ei:                      # sf of the wrong dtype
        mr.moe_reduce_fused(x, pos, w, sf=torch.ones(4, device=DEV, dtype=torch.float16))
    assert ei.value.status == 3


def test_reduce_fp8_decodes_every_code():
    # K = 1, unit weight, fp32 out: y is the decoded row itself, so all 256
    # codes (both NaN patterns, both zeros, subnormals, +-448) are compared
    # with the oracle's decode of the E4M3 format.
    mr = _mr()
    codes = torch.arange(256, dtype=torch.uint8).repeat(4).view(4, 256)
    x = codes.view(torch.float8_e4m3fn).to(DEV)
    pos = torch.arange(4, device=DEV, dtype=torch.int32).view(4, 1)
    y = mr.moe_reduce_fused(x, pos, None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    ref = oracle.to_f32(codes.numpy(), oracle.FP8) + np.float32(0.0)    # fma onto +0
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_reduce_fp8_encodes_every_code_and_tie():
    # K = 1, unit weight, fp32 in, FP8 out: y is the E4M3 encoding of the
    # input row itself. Inputs: the value of every finite code, the midpoint
    # of every pair of neighbouring codes (a tie, which goes to the even
    # code), one fp32 ulp either side of each midpoint, magnitudes at and
    # past 448 and infinities (saturate to +-448), values below half the
    # smallest subnormal (to zero), NaN; both signs (NaN positive only: the
    # fp32 multiply-add in front of the store does not keep a NaN's sign).
    # Compared bit for bit with the oracle's encoder.
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.to_f32(codes, oracle.FP8)
    fin = np.unique(vals[~np.isnan(vals) & (vals >= 0)]).astype(np.float32)
    mids = ((fin[:-1].astype(np.float64) + fin[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64) * 2, fin[:-1].astype(np.float64) + fin[1:])
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    extra = np.array([448, 449, 463.9, 464, 465, 480, 1e6, 3e38, np.inf,
                      2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -10, 2.0 ** -20], np.float32)
    pos_vals = np.concatenate([fin, mids, up, dn, extra])
    allv = np.concatenate([pos_vals, -pos_vals, np.array([np.nan], np.float32)])
    H = 256
    allv = np.concatenate([allv, np.zeros((-len(allv)) % H, np.float32)])
    x = torch.from_numpy(allv.reshape(-1, H).copy()).to(DEV)
    R = x.shape[0]
    pos = torch.arange(R, device=DEV, dtype=torch.int32).view(R, 1)
    _check_scaled(x, pos, None, None, None, torch.float8_e4m3fn)
