"""Pins for the oracle's W4A8 functions (CPU only): int4 weights packed two
per byte with int8 activations and int32 accumulation (the tutorial's
w4a8_dequant_gemm skeleton), the per-row quantizers, and the forward with
W4A8 experts.

  * the GEMM against numpy's int64 matmul over weights unpacked with the
    skeleton's own recipe (shift the field down, mask it, shift it up into
    the top of an int8 and shift back arithmetically), a different formula
    from the oracle's two's complement reading; closed forms for constant
    nibble patterns (+1, -1, -8, 7 on even / odd positions only); the
    transposed [N, M] output; the int32 range guard;
  * the quantizers: scales amax / 127 and amax / 7 in fp32, every code the
    nearest integer to v / s (numpy's round-half-even of the fp32 quotient),
    the row maximum at +-127 / +-7, zero rows, exact round trips;
  * the forward: on inputs that every step represents exactly (integer x
    with row maximum 127, weights 2^-k x int4 with row maximum 7) the gate/up
    stage equals the 16-bit forward's bit for bit; the whole forward against
    a float64 evaluation from the dequantised operands (with the int8
    quantisation of h taken by numpy), and a masked slot contributing zero.
"""
import numpy as np
import torch

import oracle


def _page_unpack(packed):
    """int4 fields of packed uint8 [..., K/2] as int8 [..., K]: field j at
    position j % 2 of byte j // 2, sign-extended by moving it to the top of
    an int8 and shifting back arithmetically."""
    b = packed.astype(np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.int8)
    for pos in (0, 1):
        field = (b >> np.uint8(4 * pos)) & np.uint8(0xF)
        top = (field << np.uint8(4)).astype(np.uint8).view(np.int8)
        out[..., pos::2] = top >> np.int8(4)
    return out


def _pack(vals):
    """int4 values [..., K] in [-8, 7] -> packed uint8 [..., K/2] (element
    2i low nibble) -- built with integer arithmetic on the two's complement."""
    v = (np.asarray(vals, np.int64) % 16).astype(np.uint8)
    return (v[..., 0::2] | (v[..., 1::2] << 4)).astype(np.uint8)


def test_gemm_against_numpy_matmul():
    rng = np.random.default_rng(0)
    M, N, K = 7, 40, 512
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    Ct = oracle.w4a8_gemm(A, B)
    ref = _page_unpack(B).astype(np.int64) @ A.astype(np.int64).T          # [N, M]
    assert Ct.shape == (N, M) and Ct.dtype == np.int32
    assert np.array_equal(Ct, ref)


def test_gemm_closed_forms():
    rng = np.random.default_rng(1)
    M, N, K = 5, 6, 256
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    a = A.astype(np.int64)
    cases = {0x11: a.sum(1), 0xFF: -a.sum(1), 0x88: -8 * a.sum(1),
             0x07: 7 * a[:, 0::2].sum(1), 0x70: 7 * a[:, 1::2].sum(1), 0x00: 0 * a.sum(1)}
    for byte, want in cases.items():
        B = np.full((N, K // 2), byte, np.uint8)
        Ct = oracle.w4a8_gemm(A, B)
        assert np.array_equal(Ct, np.tile(want, (N, 1))), hex(byte)


def test_gemm_transposed_output():
    # B row n holds the constant n - 4 (in [-4, 1]): Ct[n, m] = (n - 4) * rowsum(A[m])
    rng = np.random.default_rng(2)
    M, N, K = 3, 6, 64
    A = rng.integers(-50, 50, size=(M, K)).astype(np.int8)
    B = _pack(np.repeat((np.arange(N) - 4)[:, None], K, axis=1))
    Ct = oracle.w4a8_gemm(A, B)
    want = (np.arange(N) - 4)[:, None] * A.astype(np.int64).sum(1)[None, :]
    assert np.array_equal(Ct, want)


def test_gemm_int32_range_guard():
    K = 2_200_000                                             # 127 * 8 * K > 2^31
    A = np.full((1, K), -127, np.int8)
    B = np.full((1, K // 2), 0x88, np.uint8)                  # all -8
    Ct = np.empty((1, 1), np.int32)
    rc = oracle.lib().oracle_w4a8_gemm(A.ctypes.data, B.ctypes.data, 1, 1, K, Ct.ctypes.data)
    assert rc == -2


def _nearest_codes(v, s, lo, hi):
    return np.clip(np.round(v.astype(np.float32) / np.float32(s)), lo, hi)


def test_quantize_int8_rows():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((6, 200)) * rng.uniform(0.01, 5, size=(6, 1))).astype(np.float32)
    a[2] = 0.0
    q, s = oracle.quantize_int8_rows(oracle.F32, a)
    amax = np.abs(a).max(1)
    for r in range(6):
        if r == 2:
            assert s[r] == 1.0 and np.all(q[r] == 0)
            continue
        assert s[r] == np.float32(amax[r]) / np.float32(127.0)
        assert np.array_equal(q[r], _nearest_codes(a[r], s[r], -127, 127))
        assert np.abs(q[r]).max() == 127


def test_quantize_int8_rows_exact_round_trip():
    rng = np.random.default_rng(4)
    codes = rng.integers(-127, 128, size=(4, 96))
    codes[:, 0] = 127
    a = (codes * 2.0 ** -3).astype(np.float32)
    q, s = oracle.quantize_int8_rows(oracle.F32, a)
    assert np.all(s == np.float32(2.0 ** -3))
    assert np.array_equal(q.astype(np.int64), codes)


def test_quantize_int4_rows():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((5, 64)) * rng.uniform(0.01, 3, size=(5, 1))).astype(np.float32)
    w[4] = 0.0
    packed, s = oracle.quantize_int4_rows(oracle.F32, w)
    assert packed.shape == (5, 32)
    q = _page_unpack(packed)
    amax = np.abs(w).max(1)
    for r in range(4):
        assert s[r] == np.float32(amax[r]) / np.float32(7.0)
        assert np.array_equal(q[r], _nearest_codes(w[r], s[r], -8, 7))
        assert np.abs(q[r]).max() == 7
    assert s[4] == 1.0 and np.all(packed[4] == 0)


def test_quantize_int4_rows_exact_round_trip():
    rng = np.random.default_rng(6)
    codes = rng.integers(-7, 8, size=(3, 128))
    codes[:, 5] = -7                                          # the row maximum |7|
    w = (codes * 2.0 ** -6).astype(np.float32)
    packed, s = oracle.quantize_int4_rows(oracle.F32, w)
    assert np.all(s == np.float32(2.0 ** -6))
    assert np.array_equal(packed, _pack(codes))


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _exact_weights(rng, shape):
    """2^-k x int4 codes with a row maximum of 7 (k per row): exact in bf16
    and reproduced exactly by the int4 quantizer."""
    c = rng.integers(-7, 8, size=shape)
    c[..., 0] = 7
    k = rng.integers(4, 9, size=shape[:-1])
    return (c * 2.0 ** (-k[..., None])).astype(np.float32)


def _routing(rng, T, E, K):
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    return ids, w


def test_forward_gate_up_equals_16bit_forward_on_exact_inputs():
    rng = np.random.default_rng(7)
    T, H, D, E, K = 9, 64, 32, 3, 2
    x = rng.integers(-127, 128, size=(T, H)).astype(np.float32)
    x[:, 3] = 127.0                                           # s_x = 1 exactly
    wg, wu, wd = (_exact_weights(rng, sh) for sh in ((E, D, H), (E, D, H), (E, H, D)))
    ids, w = _routing(rng, T, E, K)
    ids[4, 1] = -1
    q = [oracle.quantize_int4_rows(oracle.F32, a) for a in (wg, wu, wd)]
    bits = [_bf16_bits(a) for a in (x, wg, wu, wd)]
    _, h16, _ = oracle.moe_forward(oracle.BF16, *bits, ids, w, want_pairs=True)
    _, h4, e4 = oracle.moe_forward_w4a8(oracle.BF16, bits[0], q[0][0], q[1][0], q[2][0], q[0][1],
                                        q[1][1], q[2][1], ids, w, want_pairs=True)
    assert np.array_equal(h4, h16)
    assert np.all(h4[4 * K + 1] == 0) and np.all(e4[4 * K + 1] == 0)   # the masked slot


def test_forward_against_float64_evaluation():
    rng = np.random.default_rng(8)
    T, H, D, E, K = 12, 128, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = _bf16_bits(x)
    ws = [(rng.standard_normal(sh) / np.sqrt(sh[-1])).astype(np.float32)
          for sh in ((E, D, H), (E, D, H), (E, H, D))]
    q = [oracle.quantize_int4_rows(oracle.F32, a) for a in ws]
    deq = [_page_unpack(p).astype(np.float64) * s[..., None].astype(np.float64) for p, s in q]
    ids, w = _routing(rng, T, E, K)
    ids[3, 0] = -1
    y = oracle.moe_forward_w4a8(oracle.BF16, xb, q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                                q[2][1], ids, w)
    xf = oracle.to_f32(xb, oracle.BF16)
    ref = np.zeros((T, H))
    for t in range(T):
        sx = np.float32(np.abs(xf[t]).max()) / np.float32(127.0)
        xq = np.clip(np.round(xf[t] / sx), -127, 127).astype(np.float64) * np.float64(sx)
        for k in range(K):
            e = ids[t, k]
            if e < 0:
                continue
            g = deq[0][e] @ xq
            u = deq[1][e] @ xq
            h = _bf16_round(g / (1 + np.exp(-g)) * u)
            sh = np.float32(np.abs(h).max()) / np.float32(127.0)
            hq = np.clip(np.round(h / sh), -127, 127).astype(np.float64) * np.float64(sh)
            eo = _bf16_round(deq[2][e] @ hq).astype(np.float64)
            ref[t] += w[t, k] * eo
    diff = y - ref
    # fp32 vs float64 epilogues and bf16 roundings only, plus the rare int8
    # code of h that lands on the other side of a rounding boundary
    assert np.abs(diff).max() <= 2e-2
    assert np.linalg.norm(diff) / np.linalg.norm(ref) <= 2e-3
