"""Pins for the oracle's block-scaled (MX) functions (CPU only): MXFP4 /
MXFP8 quantisation with one E8M0 scale per 32-element block, decoding, and
the forward with MXFP4 expert weights against MXFP8 activations.

  * E2M1 decoding against the element table built from the format
    definition (sign, 2 exponent bits with bias 1, 1 mantissa bit, exponent
    0 subnormal); E4M3 against the grid of all finite values;
  * the quantizer: the shared exponent floor(log2 amax) - emax_elem (numpy's
    log2), every element the grid value nearest to v / X with the tie cases
    of the E2M1 grid going to the even code, saturation, zero blocks, exact
    round trips of representable blocks;
  * the forward: with every value exactly representable (so every product
    and sum is exact in fp32) its gate/up stage equals the 16-bit forward's
    bit for bit; against a float64 evaluation of the same steps.
"""
import numpy as np
import torch

import oracle

FP4 = oracle.MX_FP4
FP8 = oracle.MX_FP8


def _e2m1_table():
    vals = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = 0.5 * m if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        vals.append(-mag if s else mag)
    return np.array(vals)


E2M1 = _e2m1_table()
E2M1_POS = np.unique(np.abs(E2M1))                      # 0 .. 6


def _e4m3_pos():
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if not (e == 15 and m == 7):
                vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.unique(vals)


E4M3_POS = _e4m3_pos()


def _pack4(codes):
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_e2m1_decoding():
    codes = _pack4(np.tile(np.arange(16), 2)[None])      # one block of 32: every code twice
    scales = np.full((1, 1), 127, np.uint8)              # X = 1
    dec = oracle.mx_decode(codes, scales, FP4)[0]
    assert np.array_equal(dec, np.tile(E2M1, 2).astype(np.float32))
    assert sorted(set(np.abs(E2M1))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _nearest(grid, q):
    """Nearest grid magnitude to |q| (numpy), ties to the even grid index."""
    a = np.abs(q).astype(np.float64)
    out = np.empty_like(a)
    for i, x in enumerate(a.ravel()):
        d = np.abs(grid - x)
        best = np.flatnonzero(d == d.min())
        out.ravel()[i] = grid[best[0] if len(best) == 1 else best[best % 2 == 0][0]]
    return np.sign(q) * out


def test_quantize_mxfp4_scale_and_nearest():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((4, 96)) * rng.uniform(0.01, 50, size=(4, 1))).astype(np.float32)
    v[2, 32:64] = 0.0                                    # a zero block
    codes, scales = oracle.quantize_mx_rows(oracle.F32, v, FP4)
    dec = oracle.mx_decode(codes, scales, FP4)
    for r in range(4):
        for b in range(3):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[r, b] == 127 and np.all(dec[r, 32 * b:32 * b + 32] == 0)
                continue
            e = int(np.floor(np.log2(amax))) - 2 + 127
            assert scales[r, b] == e
            X = 2.0 ** (e - 127)
            want = _nearest(E2M1_POS, blk.astype(np.float32) / np.float32(X)) * X
            assert np.array_equal(dec[r, 32 * b:32 * b + 32], want.astype(np.float32))


def test_quantize_mxfp4_ties_and_saturation():
    q = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, -0.25, -5.0, 4.0], np.float32)
    want = np.array([0, 1, 1, 2, 2, 4, 4, 6, 6, 0, -4, 4], np.float32)
    blk = np.zeros(32, np.float32)
    blk[:12] = q
    blk[12] = 4.0                                         # amax < 8: X = 1 (floor(log2 7) = 2)
    codes, scales = oracle.quantize_mx_rows(oracle.F32, blk[None], FP4)
    assert scales[0, 0] == 127
    assert np.array_equal(oracle.mx_decode(codes, scales, FP4)[0, :12], want)


def test_quantize_mxfp8_scale_and_nearest():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((3, 64)) * rng.uniform(1e-3, 1e3, size=(3, 1))).astype(np.float32)
    codes, scales = oracle.quantize_mx_rows(oracle.F32, v, FP8)
    dec = oracle.mx_decode(codes, scales, FP8)
    for r in range(3):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            e = int(np.floor(np.log2(np.abs(blk).max()))) - 8 + 127
            assert scales[r, b] == e
            X = 2.0 ** (e - 127)
            want = _nearest(E4M3_POS, blk.astype(np.float32) / np.float32(X)) * X
            assert np.array_equal(dec[r, 32 * b:32 * b + 32], want.astype(np.float32))


def test_quantize_mx_exact_round_trips():
    rng = np.random.default_rng(2)
    g4 = rng.choice(np.concatenate([-E2M1_POS, E2M1_POS]), size=(2, 64))
    g4[:, 0] = 6.0
    g4[:, 32] = -6.0
    v4 = (g4 * 2.0 ** -5).astype(np.float32)
    c4, s4 = oracle.quantize_mx_rows(oracle.F32, v4, FP4)
    assert np.all(s4 == 127 - 5)
    assert np.array_equal(oracle.mx_decode(c4, s4, FP4), v4)
    g8 = rng.choice(np.concatenate([-E4M3_POS, E4M3_POS]), size=(2, 64))
    g8[:, 0] = 448.0
    g8[:, 40] = 320.0                                     # second block: floor(log2 320) = 8
    v8 = (g8 * 2.0 ** 3).astype(np.float32)
    c8, s8 = oracle.quantize_mx_rows(oracle.F32, v8, FP8)
    assert np.array_equal(oracle.mx_decode(c8, s8, FP8), v8)


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _exact_blocks(rng, shape, grid, top):
    """Values = grid value x 2^-k per 32-block, each block holding `top`."""
    v = rng.choice(np.concatenate([-grid, grid]), size=shape)
    v[..., ::32] = top
    k = rng.integers(2, 7, size=shape[:-1] + (shape[-1] // 32,))
    return (v * 2.0 ** -np.repeat(k, 32, axis=-1)).astype(np.float32)


def test_forward_gate_up_equals_16bit_forward_on_exact_inputs():
    rng = np.random.default_rng(3)
    T, H, D, E, K = 8, 64, 64, 3, 2
    small = np.array([0, 1, 2, 3, 4, 6], np.float64)
    x = rng.choice(np.concatenate([-small, small]), size=(T, H)).astype(np.float32)
    x[:, ::32] = 6.0                                      # every x block: X = 2^-6, codes exact
    wg, wu, wd = (_exact_blocks(rng, sh, E2M1_POS, 6.0) for sh in ((E, D, H), (E, D, H), (E, H, D)))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[5, 1] = -1
    w = rng.uniform(0.1, 1, size=(T, K)).astype(np.float32)
    q = [oracle.quantize_mx_rows(oracle.F32, a, FP4) for a in (wg, wu, wd)]
    for (c, s), a in zip(q, (wg, wu, wd)):
        assert np.array_equal(oracle.mx_decode(c, s, FP4), a)
    bits = [_bf16_bits(a) for a in (x, wg, wu, wd)]
    _, h16, _ = oracle.moe_forward(oracle.BF16, *bits, ids, w, want_pairs=True)
    _, hm, em = oracle.moe_forward_mx(oracle.BF16, bits[0], q[0][0], q[1][0], q[2][0], q[0][1],
                                      q[1][1], q[2][1], ids, w, want_pairs=True)
    assert np.array_equal(hm, h16)
    assert np.all(hm[5 * K + 1] == 0) and np.all(em[5 * K + 1] == 0)


def test_forward_against_float64_evaluation():
    rng = np.random.default_rng(4)
    T, H, D, E, K = 10, 128, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = _bf16_bits(x)
    ws = [(rng.standard_normal(sh) / np.sqrt(sh[-1])).astype(np.float32)
          for sh in ((E, D, H), (E, D, H), (E, H, D))]
    q = [oracle.quantize_mx_rows(oracle.F32, a, FP4) for a in ws]
    deq = [oracle.mx_decode(c, s, FP4).astype(np.float64) for c, s in q]
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1, size=(T, K)).astype(np.float32)
    y = oracle.moe_forward_mx(oracle.BF16, xb, q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                              q[2][1], ids, w)
    xc, xs = oracle.quantize_mx_rows(oracle.BF16, xb, FP8)
    xq = oracle.mx_decode(xc, xs, FP8).astype(np.float64)
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            g = deq[0][e] @ xq[t]
            u = deq[1][e] @ xq[t]
            h = _bf16_round(g / (1 + np.exp(-g)) * u)
            hc, hs = oracle.quantize_mx_rows(oracle.F32, h[None], FP8)
            hq = oracle.mx_decode(hc, hs, FP8)[0].astype(np.float64)
            ref[t] += w[t, k] * _bf16_round(deq[2][e] @ hq)
    diff = y - ref
    assert np.abs(diff).max() <= 2e-2
    assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 2e-3
