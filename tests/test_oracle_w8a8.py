"""Pins for the oracle's W8A8 forward (CPU only): FP8 E4M3 expert weights with
per-row scales against FP8 E4M3 activations with per-row scales (x per
token, h per routed pair), the weight + activation mode of the tutorial's
module docstring.

  * on inputs every step represents exactly -- rows that are power-of-two
    scales times E4M3 values with the row maximum at 448 x scale, so both
    quantizers reproduce them exactly -- the gate/up stage equals the 16-bit
    forward's bit for bit (a power-of-two scale commutes with every fp32
    rounding, and the products are summed in the same order), so a missing,
    doubled or misplaced scale of either operand fails;
  * the whole forward against a float64 evaluation from the decoded codes
    and scales (the activation codes from the pinned per-row quantizer), with
    the bf16 roundings of h and expert_out at the same points;
  * a masked slot contributes zero, and its h / expert_out rows are zero.
"""
import numpy as np
import torch

import oracle
from test_oracle_fp8w import GRID


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _exact_rows(rng, shape):
    """Rows of 2^-k x E4M3 grid values (k per row) with a row maximum of
    448 x 2^-k: exact in bf16, and the per-row FP8 quantizer returns scale
    2^-k and the grid values as codes."""
    pos = GRID[(GRID >= 2.0 ** -3) & (GRID <= 16.0)]
    v = rng.choice(pos, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    v[..., 1] = 448.0
    k = rng.integers(2, 9, size=shape[:-1])
    return (v * 2.0 ** (-k[..., None])).astype(np.float32)


def _routing(rng, T, E, K):
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    return ids, w


def test_quantizer_reproduces_exact_rows():
    rng = np.random.default_rng(3)
    a = _exact_rows(rng, (5, 64))
    q, s = oracle.quantize_fp8_rows(oracle.F32, a)
    assert np.array_equal(oracle.to_f32(q, oracle.FP8) * s[:, None], a)
    assert np.all(np.log2(s) == np.round(np.log2(s)))


def test_gate_up_equals_16bit_forward_on_exact_inputs():
    rng = np.random.default_rng(11)
    T, H, D, E, K = 9, 64, 32, 3, 2
    x = _exact_rows(rng, (T, H))
    wg, wu, wd = (_exact_rows(rng, sh) for sh in ((E, D, H), (E, D, H), (E, H, D)))
    ids, w = _routing(rng, T, E, K)
    ids[4, 1] = -1
    q = [oracle.quantize_fp8_rows(oracle.F32, a) for a in (wg, wu, wd)]
    bits = [_bf16_bits(a) for a in (x, wg, wu, wd)]
    _, h16, _ = oracle.moe_forward(oracle.BF16, *bits, ids, w, want_pairs=True)
    _, h8, e8 = oracle.moe_forward_w8a8(oracle.BF16, bits[0], q[0][0], q[1][0], q[2][0], q[0][1],
                                        q[1][1], q[2][1], ids, w, want_pairs=True)
    assert np.array_equal(h8, h16)
    assert np.all(h8[4 * K + 1] == 0) and np.all(e8[4 * K + 1] == 0)   # the masked slot
    # The same inputs with one weight row's scale doubled in the tables
    # (codes unchanged): that row's gate values double, so h changes there.
    sg = q[0][1].copy()
    sg[ids[0, 0], 5] *= 2.0
    _, h8b, _ = oracle.moe_forward_w8a8(oracle.BF16, bits[0], q[0][0], q[1][0], q[2][0], sg,
                                        q[1][1], q[2][1], ids, w, want_pairs=True)
    assert not np.array_equal(h8b[0 * K + 0, 5], h16[0 * K + 0, 5])


def test_forward_against_float64_evaluation():
    rng = np.random.default_rng(12)
    T, H, D, E, K = 12, 128, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = _bf16_bits(x)
    ws = [(rng.standard_normal(sh) / np.sqrt(sh[-1])).astype(np.float32)
          for sh in ((E, D, H), (E, D, H), (E, H, D))]
    q = [oracle.quantize_fp8_rows(oracle.F32, a) for a in ws]
    deq = [oracle.to_f32(c, oracle.FP8).astype(np.float64) * s[..., None].astype(np.float64)
           for c, s in q]
    ids, w = _routing(rng, T, E, K)
    ids[3, 0] = -1
    y = oracle.moe_forward_w8a8(oracle.BF16, xb, q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                                q[2][1], ids, w)
    xf = oracle.to_f32(xb, oracle.BF16)
    xc, xs = oracle.quantize_fp8_rows(oracle.F32, xf)
    xq = oracle.to_f32(xc, oracle.FP8).astype(np.float64) * xs[:, None].astype(np.float64)
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            if e < 0:
                continue
            g = deq[0][e] @ xq[t]
            u = deq[1][e] @ xq[t]
            h = _bf16_round(g / (1 + np.exp(-g)) * u)
            hc, hs = oracle.quantize_fp8_rows(oracle.F32, h[None, :])
            hq = oracle.to_f32(hc[0], oracle.FP8).astype(np.float64) * np.float64(hs[0])
            eo = _bf16_round(deq[2][e] @ hq).astype(np.float64)
            ref[t] += w[t, k] * eo
    diff = y - ref
    # fp32 vs float64 sums and scale products, the bf16 roundings, and the
    # rare E4M3 code of h on the other side of a rounding boundary
    assert np.abs(diff).max() <= 2e-2
    assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 2e-3
    assert np.all(y[3] != 0)          # token 3 keeps its unmasked slot
