"""CPU oracle for the routed-expert MoE forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never loads it and shares no code with it.

Thin numpy/ctypes wrappers over ``moe_oracle.cpp``; every wrapper names the
C function it calls. Arrays are host numpy arrays. 16-bit inputs are passed
as ``uint16`` bit patterns (or numpy ``float16`` for fp16); fp32 as float32.

Dtype codes: 0 = fp16, 1 = bf16, 2 = fp32, 3 = FP8 E4M3 (OCP "fn"; reduce only).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, F32, FP8 = 0, 1, 2, 3

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = i32
        L.oracle_to_f32.argtypes = [i32, vp, f32p, i64]
        L.oracle_from_f32.argtypes = [i32, f32p, vp, i64]
        L.oracle_silu_mul.argtypes = [f32p, f32p, f32p, i64]
        L.oracle_num_blocks.argtypes = [i32, i32, i32, i32]
        L.oracle_num_blocks.restype = i64
        L.oracle_dispatch.argtypes = [i32p, f32p, i32, i32, i32, i32] + [vp] * 8
        L.oracle_dispatch.restype = i64
        L.oracle_expert_pair.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, f32p, f32p]
        L.oracle_moe_forward.argtypes = [i32, vp, vp, vp, vp, i32p, f32p, i32, i32, i32,
                                         i32, i32, i32p, i32, f32p, f32p, f32p]
        L.oracle_moe_forward_weighted_down.argtypes = L.oracle_moe_forward.argtypes
        L.oracle_reduce.argtypes = [i32, vp, i64, i32p, f32p, i32, i32, i32, f32p]
        L.oracle_reduce_scaled.argtypes = [i32, vp, i64, i32p, f32p, f32p, f32p, i32, i32, i32,
                                           f32p]
        L.oracle_quantize_fp8_rows.argtypes = [i32, vp, i64, i32, vp, f32p]
        L.oracle_moe_forward_w8.argtypes = [i32, vp, vp, vp, vp, f32p, f32p, f32p, i32p, f32p,
                                            i32, i32, i32, i32, i32, i32p, i32, f32p, f32p, f32p]
        L.oracle_gate.argtypes = [i32, vp, f32p, f32p, i32, i32, i32, i32, i32, f32p, i32p, f32p]
        L.oracle_quantize_int8_rows.argtypes = [i32, vp, i64, i32, vp, f32p]
        L.oracle_quantize_int4_rows.argtypes = [i32, vp, i64, i32, vp, f32p]
        L.oracle_w4a8_gemm.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_quantize_mx_rows.argtypes = [i32, vp, i64, i32, i32, vp, vp]
        L.oracle_mx_decode.argtypes = [vp, vp, i64, i32, i32, f32p]
        L.oracle_moe_forward_mx.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, i32p, f32p, i32, i32,
                                            i32, i32, i32, i32p, i32, f32p, f32p, f32p]
        L.oracle_moe_forward_w8a8.argtypes = [i32, vp, vp, vp, vp, f32p, f32p, f32p, i32p, f32p,
                                              i32, i32, i32, i32, i32, i32p, i32, f32p, f32p, f32p]
        L.oracle_moe_forward_w4a8.argtypes = [i32, vp, vp, vp, vp, f32p, f32p, f32p, i32p, f32p,
                                              i32, i32, i32, i32, i32, i32p, i32, f32p, f32p, f32p]
        _lib = L
    return _lib


def num_threads():
    """oracle_num_threads: OpenMP threads the oracle's loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n):
    """oracle_set_num_threads: OpenMP threads of later oracle calls."""
    assert lib().oracle_set_num_threads(int(n)) == 0


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _storage(a, dt):
    """Contiguous storage array for dtype code dt (uint8 / uint16 bits or float32)."""
    if dt == F32:
        return _c(a, np.float32)
    if dt == FP8:
        return _c(a, np.uint8)
    if a.dtype == np.float16:
        return _c(a, np.float16).view(np.uint16)
    return _c(a, np.uint16)


def to_f32(bits, dt):
    """oracle_to_f32: storage -> fp32 (exact widening)."""
    s = _storage(np.asarray(bits), dt)
    out = np.empty(s.shape, np.float32)
    assert lib().oracle_to_f32(dt, _ptr(s), _ptr(out), s.size) == 0
    return out


def from_f32(x, dt):
    """oracle_from_f32: fp32 -> storage (round to nearest even); uint16 bits for 16-bit."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, {F32: np.float32, FP8: np.uint8}.get(dt, np.uint16))
    assert lib().oracle_from_f32(dt, _ptr(x), _ptr(out), x.size) == 0
    return out


def silu_mul(g, u):
    """oracle_silu_mul: SiLU(g) * u in fp32."""
    g, u = _c(g, np.float32), _c(u, np.float32)
    out = np.empty(g.shape, np.float32)
    lib().oracle_silu_mul(_ptr(g), _ptr(u), _ptr(out), g.size)
    return out


def num_blocks(T, K, E, BM):
    return int(lib().oracle_num_blocks(T, K, E, BM))


def dispatch(ids, w, E, BM):
    """oracle_dispatch: expert-sorted tables for ids/w of shape [T, K].

    Returns a dict of numpy arrays plus ``n_valid``; raises on invalid ids.
    """
    ids = _c(ids, np.int32)
    T, K = ids.shape
    w = None if w is None else _c(w, np.float32)
    P = T * K
    nb = num_blocks(T, K, E, BM)
    out = dict(
        group_sizes=np.empty(E, np.int32), group_offsets=np.empty(E, np.int32),
        group_padded_offsets=np.empty(E, np.int32), block_expert=np.empty(nb, np.int32),
        sorted_pair=np.empty(P, np.int32), sorted_token=np.empty(P, np.int32),
        sorted_weight=np.empty(P, np.float32), token_topk_to_pos=np.empty(P, np.int32))
    n = lib().oracle_dispatch(
        _ptr(ids), _ptr(w), T, K, E, BM, _ptr(out["group_sizes"]), _ptr(out["group_offsets"]),
        _ptr(out["group_padded_offsets"]), _ptr(out["block_expert"]), _ptr(out["sorted_pair"]),
        _ptr(out["sorted_token"]), _ptr(out["sorted_weight"]), _ptr(out["token_topk_to_pos"]))
    if n < 0:
        raise ValueError("oracle_dispatch rejected its arguments")
    out["n_valid"] = int(n)
    out["token_topk_to_pos"] = out["token_topk_to_pos"].reshape(T, K)
    return out


def expert_pair(dt, x, wg, wu, wd, token, expert):
    """oracle_expert_pair: (h [D], expert_out [H]) of one pair, fp32 after rounding."""
    x, wg, wu, wd = (_storage(a, dt) for a in (x, wg, wu, wd))
    H = x.shape[-1]
    D = wg.shape[1]
    h = np.empty(D, np.float32)
    eo = np.empty(H, np.float32)
    rc = lib().oracle_expert_pair(dt, _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), int(token),
                                  int(expert), H, D, _ptr(h), _ptr(eo))
    assert rc == 0
    return h, eo


def moe_forward(dt, x, wg, wu, wd, ids, w, tokens=None, want_pairs=False, weighted_down=False):
    """oracle_moe_forward: y [n_tokens, H] fp32 (and per-slot h / expert_out).

    x [T, H]; wg, wu [E, D, H]; wd [E, H, D] (storage of dtype dt);
    ids int32 [T, K]; w fp32 [T, K]; tokens: optional token subset.
    weighted_down: oracle_moe_forward_weighted_down (the routing weight
    applied to the down output before its rounding, an unweighted combine).
    """
    x, wg, wu, wd = (_storage(a, dt) for a in (x, wg, wu, wd))
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, H = x.shape
    E, D, _ = wg.shape
    K = ids.shape[1]
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tok is None else tok.size
    y = np.empty((n, H), np.float32)
    hp = np.empty((n * K, D), np.float32) if want_pairs else None
    ep = np.empty((n * K, H), np.float32) if want_pairs else None
    fn = lib().oracle_moe_forward_weighted_down if weighted_down else lib().oracle_moe_forward
    rc = fn(dt, _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(ids), _ptr(w), T, H, D, E, K,
            _ptr(tok), n, _ptr(y), _ptr(hp), _ptr(ep))
    if rc != 0:
        raise ValueError("oracle_moe_forward rejected its arguments")
    return (y, hp, ep) if want_pairs else y


def reduce(dt, X, pos, w=None, x_sf=None, sf=None):
    """oracle_reduce / oracle_reduce_scaled: y [T, H] fp32 =
    sf[t] * sum_k (w[t,k] * x_sf[pos[t,k]]) * X[pos[t,k]] over pos >= 0."""
    X = _storage(X, dt)
    pos = _c(pos, np.int32)
    T, K = pos.shape
    R, H = X.shape
    w = None if w is None else _c(w, np.float32)
    y = np.empty((T, H), np.float32)
    if x_sf is None and sf is None:
        rc = lib().oracle_reduce(dt, _ptr(X), R, _ptr(pos), _ptr(w), T, K, H, _ptr(y))
    else:
        xs = None if x_sf is None else _c(x_sf, np.float32)
        s = None if sf is None else _c(sf, np.float32)
        rc = lib().oracle_reduce_scaled(dt, _ptr(X), R, _ptr(pos), _ptr(w), _ptr(xs), _ptr(s),
                                        T, K, H, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_reduce rejected its arguments")
    return y


def gate(dt, x, wr, K, renorm, bias=None):
    """oracle_gate: router logits (fp32 fma chain, h ascending, plus an
    optional per-expert bias), top-K by logit (ties to the lower index),
    softmax scores, optional renormalisation. x: [T, H] storage of dtype dt;
    wr: [E, H] float32; bias: [E] float32 or None. Returns dict of logits
    [T, E] float32, ids [T, K] int32, weights [T, K] float32."""
    xs = _storage(np.asarray(x), dt)
    T, H = xs.shape
    wr = _c(wr, np.float32)
    E = wr.shape[0]
    assert wr.shape == (E, H)
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    b = None if bias is None else _c(bias, np.float32)
    assert b is None or b.shape == (E,)
    rc = lib().oracle_gate(dt, _ptr(xs), _ptr(wr), _ptr(b), T, H, E, K, int(bool(renorm)),
                           _ptr(logits), _ptr(ids), _ptr(w))
    assert rc == 0, "oracle_gate rejected its arguments"
    return dict(logits=logits, ids=ids, weights=w)


def quantize_fp8_rows(dt, w):
    """oracle_quantize_fp8_rows: per-row FP8 E4M3 codes and fp32 scales
    (scale = amax / 448, 1 for a zero row). w: [..., cols] storage of dtype
    dt. Returns (codes uint8 of w's shape, scales float32 of w's shape[:-1])."""
    ws = _storage(np.asarray(w), dt)
    cols = ws.shape[-1]
    rows = ws.size // cols
    q = np.empty(ws.shape, np.uint8)
    s = np.empty(ws.shape[:-1], np.float32)
    assert lib().oracle_quantize_fp8_rows(dt, _ptr(ws), rows, cols, _ptr(q), _ptr(s)) == 0
    return q, s


def moe_forward_w8(dt, x, wg8, wu8, wd8, sg, su, sd, ids, w, tokens=None, want_pairs=False):
    """oracle_moe_forward_w8: the forward with FP8 expert weights (uint8 codes
    [E, D, H] / [E, D, H] / [E, H, D]) and per-row fp32 scales ([E, D],
    [E, D], [E, H]). Same outputs as moe_forward."""
    xs = _storage(x, dt)
    T, H = xs.shape
    E, D, _ = wg8.shape
    K = ids.shape[1]
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tokens is None else len(tok)
    y = np.empty((n, H), np.float32)
    hp = np.empty((n * K, D), np.float32) if want_pairs else None
    ep = np.empty((n * K, H), np.float32) if want_pairs else None
    args = [_c(a, np.uint8) for a in (wg8, wu8, wd8)] + [_c(a, np.float32) for a in (sg, su, sd)]
    rc = lib().oracle_moe_forward_w8(dt, _ptr(xs), *[_ptr(a) for a in args], _ptr(ids), _ptr(w),
                                     T, H, D, E, K, _ptr(tok), n, _ptr(y), _ptr(hp), _ptr(ep))
    assert rc == 0, "oracle_moe_forward_w8 rejected its arguments"
    return (y, hp, ep) if want_pairs else y


def quantize_int8_rows(dt, a):
    """oracle_quantize_int8_rows: per-row int8 codes in [-127, 127] and fp32
    scales (amax / 127, 1 for a zero row). a: [..., cols] storage of dtype dt.
    Returns (codes int8 of a's shape, scales float32 of a's shape[:-1])."""
    s_ = _storage(np.asarray(a), dt)
    cols = s_.shape[-1]
    rows = s_.size // cols
    q = np.empty(s_.shape, np.int8)
    sc = np.empty(s_.shape[:-1], np.float32)
    assert lib().oracle_quantize_int8_rows(dt, _ptr(s_), rows, cols, _ptr(q), _ptr(sc)) == 0
    return q, sc


def quantize_int4_rows(dt, w):
    """oracle_quantize_int4_rows: per-row int4 codes in [-8, 7] (amax / 7
    scales, 1 for a zero row), packed two per byte, element 2i in the low
    nibble. w: [..., cols] (cols even). Returns (packed uint8 [..., cols/2],
    scales float32 of w's shape[:-1])."""
    ws = _storage(np.asarray(w), dt)
    cols = ws.shape[-1]
    rows = ws.size // cols
    q = np.empty(ws.shape[:-1] + (cols // 2,), np.uint8)
    sc = np.empty(ws.shape[:-1], np.float32)
    assert lib().oracle_quantize_int4_rows(dt, _ptr(ws), rows, cols, _ptr(q), _ptr(sc)) == 0
    return q, sc


def w4a8_gemm(A, B):
    """oracle_w4a8_gemm: Ct [N, M] int32 = sum_k A[m, k] * B4[n, k], A int8
    [M, K], B packed int4 uint8 [N, K/2]."""
    A = _c(A, np.int8)
    B = _c(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] * 2 == K
    Ct = np.empty((N, M), np.int32)
    rc = lib().oracle_w4a8_gemm(_ptr(A), _ptr(B), M, N, K, _ptr(Ct))
    assert rc == 0, "oracle_w4a8_gemm: rejected arguments or int32 overflow (%d)" % rc
    return Ct


def moe_forward_w4a8(dt, x, wg4, wu4, wd4, sg, su, sd, ids, w, tokens=None, want_pairs=False):
    """oracle_moe_forward_w4a8: the forward with int4 expert weights (packed
    uint8 [E, D, H/2] / [E, D, H/2] / [E, H, D/2], fp32 row scales [E, D] /
    [E, D] / [E, H]) and int8 activations. Same outputs as moe_forward."""
    xs = _storage(x, dt)
    T, H = xs.shape
    E, D, _ = wg4.shape
    K = ids.shape[1]
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tokens is None else len(tok)
    y = np.empty((n, H), np.float32)
    hp = np.empty((n * K, D), np.float32) if want_pairs else None
    ep = np.empty((n * K, H), np.float32) if want_pairs else None
    args = [_c(a, np.uint8) for a in (wg4, wu4, wd4)] + [_c(a, np.float32) for a in (sg, su, sd)]
    rc = lib().oracle_moe_forward_w4a8(dt, _ptr(xs), *[_ptr(a) for a in args], _ptr(ids), _ptr(w),
                                       T, H, D, E, K, _ptr(tok), n, _ptr(y), _ptr(hp), _ptr(ep))
    assert rc == 0, "oracle_moe_forward_w4a8 rejected its arguments"
    return (y, hp, ep) if want_pairs else y


def moe_forward_w8a8(dt, x, wg8, wu8, wd8, sg, su, sd, ids, w, tokens=None, want_pairs=False):
    """oracle_moe_forward_w8a8: FP8 E4M3 expert weights (codes [E, D, H] /
    [E, D, H] / [E, H, D], fp32 row scales [E, D] / [E, D] / [E, H]) against
    FP8 E4M3 activations (x per token, h per routed pair, scale amax / 448).
    Same outputs as moe_forward."""
    xs = _storage(x, dt)
    T, H = xs.shape
    E, D, _ = wg8.shape
    K = ids.shape[1]
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tokens is None else len(tok)
    y = np.empty((n, H), np.float32)
    hp = np.empty((n * K, D), np.float32) if want_pairs else None
    ep = np.empty((n * K, H), np.float32) if want_pairs else None
    args = [_c(a, np.uint8) for a in (wg8, wu8, wd8)] + [_c(a, np.float32) for a in (sg, su, sd)]
    rc = lib().oracle_moe_forward_w8a8(dt, _ptr(xs), *[_ptr(a) for a in args], _ptr(ids), _ptr(w),
                                       T, H, D, E, K, _ptr(tok), n, _ptr(y), _ptr(hp), _ptr(ep))
    assert rc == 0, "oracle_moe_forward_w8a8 rejected its arguments"
    return (y, hp, ep) if want_pairs else y


MX_FP8, MX_FP4 = 0, 4


def quantize_mx_rows(dt, v, fmt):
    """oracle_quantize_mx_rows: MX codes and E8M0 scales (blocks of 32 along
    the last axis). fmt MX_FP8 -> E4M3 codes of v's shape; MX_FP4 -> packed
    E2M1 [..., cols/2]. Returns (codes uint8, scales uint8 [..., cols/32])."""
    vs = _storage(np.asarray(v), dt)
    cols = vs.shape[-1]
    rows = vs.size // cols
    cshape = vs.shape if fmt == MX_FP8 else vs.shape[:-1] + (cols // 2,)
    codes = np.empty(cshape, np.uint8)
    scales = np.empty(vs.shape[:-1] + (cols // 32,), np.uint8)
    assert lib().oracle_quantize_mx_rows(dt, _ptr(vs), rows, cols, fmt, _ptr(codes), _ptr(scales)) == 0
    return codes, scales


def mx_decode(codes, scales, fmt):
    """oracle_mx_decode: the fp32 values X * element of MX rows."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    cols = scales.shape[-1] * 32
    rows = scales.size // scales.shape[-1]
    out = np.empty(scales.shape[:-1] + (cols,), np.float32)
    assert lib().oracle_mx_decode(_ptr(codes), _ptr(scales), rows, cols, fmt, _ptr(out)) == 0
    return out


def moe_forward_mx(dt, x, wg, wu, wd, sg, su, sd, ids, w, tokens=None, want_pairs=False):
    """oracle_moe_forward_mx: MXFP4 expert weights (packed [E, D, H/2] /
    [E, D, H/2] / [E, H, D/2], E8M0 scales [E, D, H/32] / [E, D, H/32] /
    [E, H, D/32]) against MXFP8 activations. Same outputs as moe_forward."""
    xs = _storage(x, dt)
    T, H = xs.shape
    E, D, _ = wg.shape
    K = ids.shape[1]
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tokens is None else len(tok)
    y = np.empty((n, H), np.float32)
    hp = np.empty((n * K, D), np.float32) if want_pairs else None
    ep = np.empty((n * K, H), np.float32) if want_pairs else None
    args = [_c(a, np.uint8) for a in (wg, wu, wd, sg, su, sd)]
    rc = lib().oracle_moe_forward_mx(dt, _ptr(xs), *[_ptr(a) for a in args], _ptr(ids), _ptr(w),
                                     T, H, D, E, K, _ptr(tok), n, _ptr(y), _ptr(hp), _ptr(ep))
    assert rc == 0, "oracle_moe_forward_mx rejected its arguments"
    return (y, hp, ep) if want_pairs else y
