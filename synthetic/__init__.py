"""Seeded synthetic inputs for the routed-expert MoE forward.

This module is shared by the oracle-side and the GPU-side tests and by the
benchmark. It holds no arithmetic of the method itself (no dispatch, no
expert MLP, no SiLU, no weighted reduce): only a counter-based random number
generator, the workload shapes, and the router that turns tokens into top-k
expert ids and weights (the router sits before the MoE forward and is not
part of it).

Generator: SplitMix64's output function applied to a 64-bit counter
(key(seed, stream) + (i + 1) * golden-ratio constant, mod 2^64), the
published SplitMix64 construction (Steele, Lea, Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014). Uniforms take the top 53 bits
as (b + 0.5) * 2^-53; normals use Box-Muller (cosine branch) on the uniforms
of counters 2i and 2i + 1. Every value depends only on (seed, stream, index),
never on the device, chunking or thread count (up to the last ulp of the
float64 log/cos, which the final rounding to 16 bits absorbs in practice).
Torch is used as an array library so the same code runs on CPU and GPU.
"""
import math

import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# Tensor streams (one per tensor so that shapes can change independently).
S_X, S_ROUTER, S_GATE, S_UP, S_DOWN = 1, 2, 3, 4, 5
S_RED_X, S_RED_W, S_RED_PERM, S_RED_MASK = 6, 7, 8, 9

_CHUNK = 1 << 24

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _s64(v):
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_py(z):
    """SplitMix64 output function on a Python int (reference for the tensor form)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def _srl(z, s):
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z):
    z = (z ^ _srl(z, 30)) * _s64(MIX1)
    z = (z ^ _srl(z, 27)) * _s64(MIX2)
    return z ^ _srl(z, 31)


def stream_key(seed, stream):
    return mix64_py(seed * GOLDEN + stream * MIX2 + 1)


def bits64(seed, stream, start, n, device="cpu"):
    """Raw 64-bit outputs (as int64 bit patterns) for counters start..start+n-1."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    z = (idx + 1) * _s64(GOLDEN) + _s64(stream_key(seed, stream))
    return _mix64(z)


def _uniform_from_bits(b):
    return (_srl(b, 11).to(torch.float64) + 0.5) * (2.0 ** -53)


def uniform(seed, stream, start, n, device="cpu"):
    """U(0,1) float64 for counters start..start+n-1."""
    return _uniform_from_bits(bits64(seed, stream, start, n, device))


def _normal_chunk(seed, stream, start, n, device):
    b = bits64(seed, stream, 2 * start, 2 * n, device).view(n, 2)
    u1 = _uniform_from_bits(b[:, 0])
    u2 = _uniform_from_bits(b[:, 1])
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def normal(shape, std, seed, stream, dtype, device="cpu"):
    """N(0, std^2) tensor of `dtype`; computed in float64, rounded via float32."""
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=dtype, device=device)
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        z = _normal_chunk(seed, stream, start, m, device) * std
        out[start:start + m] = z.to(torch.float32).to(dtype)
    return out.view(*shape)


def uniform_tensor(shape, seed, stream, device="cpu"):
    n = 1
    for s in shape:
        n *= s
    return uniform(seed, stream, 0, n, device).to(torch.float32).view(*shape)


# ------------------------------------------------------------- workloads --

CONFIGS = [
    dict(name="tiny-f16", dtype="f16", T=64, H=256, D=128, E=8, K=2,
         renorm=False, zipf=False, seed=0),
    dict(name="mid-bf16", dtype="bf16", T=512, H=2048, D=768, E=128, K=8,
         renorm=True, zipf=False, seed=1),
    dict(name="deepseek-decode-bf16", dtype="bf16", T=512, H=7168, D=2048, E=256, K=8,
         renorm=True, zipf=False, seed=2),
    dict(name="deepseek-prefill-bf16", dtype="bf16", T=4096, H=7168, D=2048, E=256, K=8,
         renorm=True, zipf=False, seed=3),
    dict(name="skewed-prefill-bf16", dtype="bf16", T=4096, H=7168, D=2048, E=256, K=8,
         renorm=True, zipf=True, seed=4),
]

ROUTER_STD = 0.02


def route(x, router, K, renorm, bias=None):
    """Top-k routing (the gate that precedes the MoE forward).

    logits = x . router^T (computed in float64 from the already-rounded x,
    then taken to fp32), optional additive bias, fp32 softmax, top-k by
    probability with ties going to the lower expert index, weights = the
    selected probabilities, optionally renormalised to sum to one.
    Returns (ids int32 [T, K], weights fp32 [T, K]).
    """
    logits = (x.to(torch.float64) @ router.to(torch.float64).t()).to(torch.float32)
    if bias is not None:
        logits = logits + bias.to(logits.device)
    probs = torch.softmax(logits, dim=-1)
    order = torch.sort(probs, dim=-1, descending=True, stable=True).indices[:, :K]
    w = probs.gather(1, order)
    if renorm:
        w = w / w.sum(dim=-1, keepdim=True)
    return order.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


def zipf_bias(E):
    """Additive router-logit bias 2*log(1/rank) with rank(e) = e + 1."""
    return (-2.0 * torch.log(torch.arange(1, E + 1, dtype=torch.float64))).to(torch.float32)


def make_moe_inputs(cfg, device="cpu", T=None, seed=None, weights=True):
    """Inputs of one routed-MoE workload.

    x ~ N(0, 1) and expert weights ~ N(0, 1/fan_in) (fan_in = H for gate/up,
    D for down), all rounded to the workload dtype; router ~ N(0, 0.02^2) fp32.
    `T` overrides the token count (same generators, a prefix of the tokens).
    """
    dt = DTYPES[cfg["dtype"]]
    seed = cfg["seed"] if seed is None else seed
    T = cfg["T"] if T is None else T
    H, D, E, K = cfg["H"], cfg["D"], cfg["E"], cfg["K"]
    x = normal((T, H), 1.0, seed, S_X, dt, device)
    router = normal((E, H), ROUTER_STD, seed, S_ROUTER, torch.float32, device)
    bias = zipf_bias(E) if cfg.get("zipf") else None
    ids, w = route(x, router, K, cfg["renorm"], bias)
    out = dict(x=x, router=router, topk_ids=ids, topk_weights=w, dtype=dt,
               T=T, H=H, D=D, E=E, K=K)
    if weights:
        out["w_gate"] = normal((E, D, H), 1.0 / math.sqrt(H), seed, S_GATE, dt, device)
        out["w_up"] = normal((E, D, H), 1.0 / math.sqrt(H), seed, S_UP, dt, device)
        out["w_down"] = normal((E, H, D), 1.0 / math.sqrt(D), seed, S_DOWN, dt, device)
    return out


def make_reduce_inputs(T, K, H, dtype="bf16", seed=4, mask_frac=0.1, device="cpu", R=None,
                       rows=True):
    """Inputs of a standalone weighted reduce.

    expert_out [R, H] ~ N(0, 1) (R = T*K by default; None when rows=False);
    topk_weights [T, K] ~ U(0, 1) normalised per row over all K slots;
    token_topk_to_pos = a seeded random permutation of [0, T*K) (taken mod R
    when R < T*K) with floor(mask_frac * T * K) seeded slots set to -1.
    """
    dt = DTYPES[dtype]
    P = T * K
    R = P if R is None else R
    x = normal((R, H), 1.0, seed, S_RED_X, dt, device) if rows else None
    w = uniform_tensor((T, K), seed, S_RED_W, device)
    w = (w / w.sum(dim=-1, keepdim=True)).contiguous()
    perm_keys = bits64(seed, S_RED_PERM, 0, P, device)
    pos = torch.argsort(perm_keys, stable=True).to(torch.int64) % R
    pos = pos.to(torch.int32)
    n_mask = int(math.floor(mask_frac * P))
    if n_mask:
        mask_keys = bits64(seed, S_RED_MASK, 0, P, device)
        masked = torch.argsort(mask_keys, stable=True)[:n_mask]
        pos[masked] = -1
    return dict(expert_out=x, token_topk_to_pos=pos.view(T, K).contiguous(),
                topk_weights=w, dtype=dt, T=T, K=K, H=H, R=R)
