"""Routed-expert MoE forward on AMD Instinct MI355X (gfx950) -- Python binding.

Argument marshalling only: every step runs in the HIP kernels of
libmoe_routed.so, called through its C ABI (include/moe_routed.h). PyTorch
supplies device memory and the current stream; the binding checks dtypes,
shapes, devices and contiguity (the C ABI sees raw pointers only) and raises
MoeError with the library's status code on any failure.

    ids, weights, logits = moe_gate(x, w_router, top_k)              # step 0
    tables = moe_dispatch(topk_ids, topk_weights, num_experts)      # step 1
    y = moe_routed_forward(x, w_gate, w_up, w_down, tables)         # steps 2-3
    y = moe_reduce_fused(expert_out, token_topk_to_pos, topk_weights)  # step 3 alone
"""
import ctypes
import math

import torch

from ._lib import (MOE_BF16, MOE_ERR_DTYPE, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_F16, MOE_F32,
                   MOE_FP8_E4M3,
                   MoeError, MoeTablesStruct, check, lib)

__all__ = ["MoeError", "MoeTables", "FP8Weights", "default_block_m", "moe_gate", "moe_dispatch",
           "quantize_fp8_rows", "moe_expert_gate_up_w8", "moe_expert_down_w8",
           "moe_routed_forward_w8", "moe_expert_gate_up",
           "moe_expert_down", "moe_routed_forward", "moe_reduce_fused", "forward_workspace",
           "moe_expert_down_weighted", "moe_routed_forward_weighted",
           "W4Weights", "quantize_int8_rows", "quantize_int4_rows", "w4a8_gemm",
           "moe_expert_gate_up_w4a8", "moe_expert_down_w4a8", "forward_w4a8_workspace",
           "moe_routed_forward_w4a8", "MX_FP8", "MX_FP4", "MXWeights", "quantize_mx_rows",
           "quantize_mx_weights", "moe_expert_gate_up_mx", "moe_expert_down_mx",
           "forward_mx_workspace", "moe_routed_forward_mx"]

MX_FP8, MX_FP4 = 0, 4

_DTYPE_CODE = {torch.float16: MOE_F16, torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}
# The reduce also reads and writes OCP FP8 E4M3 ("fn").
_REDUCE_CODE = {**_DTYPE_CODE, torch.float8_e4m3fn: MOE_FP8_E4M3}

_TABLE_FIELDS = {
    "group_sizes": ("E", torch.int32), "group_offsets": ("E", torch.int32),
    "group_padded_offsets": ("E", torch.int32), "block_expert": ("num_blocks", torch.int32),
    "sorted_pair": ("P", torch.int32), "sorted_token": ("P", torch.int32),
    "sorted_weight": ("P", torch.float32), "token_topk_to_pos": ("P", torch.int32),
    "topk_weights": ("P", torch.float32), "status": ("one", torch.int32),
    "active_blocks": ("num_blocks", torch.int32), "active_count": ("one", torch.int32),
}


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(cond, status, msg):
    if not cond:
        raise MoeError(status, msg)


def _check_tensor(t, name, dtype=None, ndim=None, device=None):
    _require(t is not None, MOE_ERR_NULL, "%s must not be None" % name)
    _require(t.is_cuda, MOE_ERR_SHAPE, "%s must be a GPU tensor" % name)
    if device is not None:
        _require(t.device == device, MOE_ERR_SHAPE, "%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None:
        _require(t.dtype == dtype, MOE_ERR_DTYPE, "%s must be %s (got %s)" % (name, dtype, t.dtype))
    if ndim is not None:
        _require(t.dim() == ndim, MOE_ERR_SHAPE, "%s must be %d-D (got shape %s)" % (name, ndim, tuple(t.shape)))
    _require(t.is_contiguous(), MOE_ERR_SHAPE, "%s must be contiguous" % name)


# Largest row block worth building for each weight format: the W4A8 and MX
# grouped kernels keep 128 / 64 rows per pass over the weights, and smaller
# blocks let an expert's row blocks run side by side on one XCD and share
# the weight reads in its L2 instead of re-reading them pass after pass
# (measured at the DeepSeek prefill shape, T = 4096: W4A8 3.30 -> 3.20 ms at
# 128, MX 3.88 -> 3.58 ms at 64).
_BLOCK_M_CAP = {"w4a8": 128, "mx": 64}


def default_block_m(T, K, E, weights="16bit"):
    """Row-block size of the tables: the power of two >= twice the mean rows
    per expert, clamped to [16, 256], so a typical expert fits in one block
    and its weights are streamed once; for W4A8 and MX weights ("w4a8",
    "mx") at most their kernels' pass height (128 / 64 rows)."""
    avg = max(1.0, T * K / E)
    bm = 1 << max(0, math.ceil(math.log2(2 * avg)))
    return int(min(256, _BLOCK_M_CAP.get(weights, 256), max(16, bm)))


class MoeTables:
    """Dispatch tables in one device buffer (struct moe_tables of the C ABI)."""

    def __init__(self, T, K, E, block_m, device):
        nbytes = lib().moe_tables_bytes(T, K, E, block_m)
        if nbytes == 0:
            # Let the library name the bad argument.
            s = MoeTablesStruct()
            check(lib().moe_tables_bind(ctypes.byref(s), ctypes.c_void_p(256), 0, T, K, E, block_m))
        self.T, self.K, self.E, self.block_m = T, K, E, block_m
        self.device = torch.device(device)
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.struct = MoeTablesStruct()
        check(lib().moe_tables_bind(ctypes.byref(self.struct), _ptr(self.buffer), nbytes,
                                    T, K, E, block_m))
        self.num_blocks = self.struct.num_blocks

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    def tensor(self, name):
        """A torch view of one table (see the header for its meaning)."""
        count, dtype = _TABLE_FIELDS[name]
        n = {"E": self.E, "num_blocks": self.num_blocks, "P": self.T * self.K, "one": 1}[count]
        off = getattr(self.struct, name) - self.buffer.data_ptr()
        raw = self.buffer[off:off + 4 * n]
        return raw.view(dtype)

    def __getattr__(self, name):
        if name in _TABLE_FIELDS:
            return self.tensor(name)
        raise AttributeError(name)


def moe_gate(x, w_router, top_k, renorm=True, bias=None, out=None):
    """Step 0: router gate. x [T, H] (fp16 / bf16 / fp32), w_router [E, H]
    float32, bias [E] float32 or None. Returns (topk_ids int32 [T, K],
    topk_weights float32 [T, K], logits float32 [T, E]); `out` may pass
    those three tensors to fill."""
    _check_tensor(x, "x", None, 2)
    _require(x.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "x must be float16, bfloat16 or float32")
    _check_tensor(w_router, "w_router", torch.float32, 2, x.device)
    T, H = x.shape
    E = w_router.shape[0]
    _require(w_router.shape[1] == H, MOE_ERR_SHAPE, "w_router must be [E, %d]" % H)
    if bias is not None:
        _check_tensor(bias, "bias", torch.float32, 1, x.device)
        _require(bias.shape[0] == E, MOE_ERR_SHAPE, "bias must be [%d]" % E)
    K = int(top_k)
    if out is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=x.device)
        w = torch.empty((T, K), dtype=torch.float32, device=x.device)
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    else:
        ids, w, logits = out
        _check_tensor(ids, "topk_ids", torch.int32, 2, x.device)
        _check_tensor(w, "topk_weights", torch.float32, 2, x.device)
        _check_tensor(logits, "logits", torch.float32, 2, x.device)
        _require(tuple(ids.shape) == (T, K) and tuple(w.shape) == (T, K)
                 and tuple(logits.shape) == (T, E), MOE_ERR_SHAPE, "output shapes do not match")
    check(lib().moe_gate(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, K, int(bool(renorm)),
                         _DTYPE_CODE[x.dtype], _ptr(logits), _ptr(ids), _ptr(w),
                         _stream(x.device)))
    return ids, w, logits


def moe_dispatch(topk_ids, topk_weights, num_experts, block_m=None, tables=None):
    """Step 1: expert-sorted dispatch tables from top-k ids [T, K] (int32,
    negative = masked slot) and weights [T, K] (float32, or None = ones)."""
    _check_tensor(topk_ids, "topk_ids", torch.int32, 2)
    T, K = topk_ids.shape
    if topk_weights is not None:
        _check_tensor(topk_weights, "topk_weights", torch.float32, 2, topk_ids.device)
        _require(tuple(topk_weights.shape) == (T, K), MOE_ERR_SHAPE,
                 "topk_weights shape %s != topk_ids shape %s" % (tuple(topk_weights.shape), (T, K)))
    if block_m is None:
        block_m = default_block_m(T, K, num_experts)
    if tables is None:
        tables = MoeTables(T, K, num_experts, block_m, topk_ids.device)
    else:
        _require((tables.T, tables.K, tables.E, tables.block_m) == (T, K, num_experts, block_m),
                 MOE_ERR_SHAPE, "tables were bound for other sizes")
    check(lib().moe_dispatch(_ptr(topk_ids), _ptr(topk_weights), tables.ref,
                             _stream(topk_ids.device)))
    return tables


def _expert_shapes(x_or_h, w_a, w_b, w_down, tables, gate_up):
    dt = x_or_h.dtype
    _require(dt in (torch.float16, torch.bfloat16, torch.float32), MOE_ERR_DTYPE,
             "expert GEMMs take float16, bfloat16 or float32 (got %s)" % dt)
    E = tables.E
    if gate_up:
        T, H = x_or_h.shape
        _require(T == tables.T, MOE_ERR_SHAPE, "x has %d tokens, tables %d" % (T, tables.T))
        _require(w_a.dim() == 3 and w_a.shape[0] == E and w_a.shape[2] == H, MOE_ERR_SHAPE,
                 "w_gate must be [E=%d, D, H=%d] (got %s)" % (E, H, tuple(w_a.shape)))
        D = w_a.shape[1]
        _require(tuple(w_b.shape) == (E, D, H), MOE_ERR_SHAPE,
                 "w_up must be [%d, %d, %d] (got %s)" % (E, D, H, tuple(w_b.shape)))
        if w_down is not None:
            _require(tuple(w_down.shape) == (E, H, D), MOE_ERR_SHAPE,
                     "w_down must be [%d, %d, %d] (got %s)" % (E, H, D, tuple(w_down.shape)))
        return H, D
    P, D = x_or_h.shape
    _require(P == tables.T * tables.K, MOE_ERR_SHAPE, "h must have T*K rows")
    _require(w_a.dim() == 3 and w_a.shape[0] == E and w_a.shape[2] == D, MOE_ERR_SHAPE,
             "w_down must be [E=%d, H, D=%d] (got %s)" % (E, D, tuple(w_a.shape)))
    return w_a.shape[1], D


def moe_expert_gate_up(x, w_gate, w_up, tables, h=None):
    """Step 2a: h [T*K, D] = SiLU(x W_gate^T) * (x W_up^T) per sorted row."""
    _check_tensor(x, "x", None, 2, tables.device)
    for n, w in (("w_gate", w_gate), ("w_up", w_up)):
        _check_tensor(w, n, x.dtype, 3, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, None, tables, True)
    if h is None:
        h = torch.empty(tables.T * tables.K, D, dtype=x.dtype, device=x.device)
    _check_tensor(h, "h", x.dtype, 2, tables.device)
    check(lib().moe_expert_gate_up(_ptr(x), _ptr(w_gate), _ptr(w_up), tables.ref, H, D,
                                   _DTYPE_CODE[x.dtype], _ptr(h), _stream(x.device)))
    return h


def _down(fn, h, w_down, tables, expert_out):
    _check_tensor(h, "h", None, 2, tables.device)
    _check_tensor(w_down, "w_down", h.dtype, 3, tables.device)
    H, D = _expert_shapes(h, w_down, None, None, tables, False)
    if expert_out is None:
        expert_out = torch.empty(tables.T * tables.K, H, dtype=h.dtype, device=h.device)
    _check_tensor(expert_out, "expert_out", h.dtype, 2, tables.device)
    check(fn(_ptr(h), _ptr(w_down), tables.ref, H, D, _DTYPE_CODE[h.dtype], _ptr(expert_out),
             _stream(h.device)))
    return expert_out


def moe_expert_down(h, w_down, tables, expert_out=None):
    """Step 2b: expert_out [T*K, H] = h W_down^T per sorted row (unweighted)."""
    return _down(lib().moe_expert_down, h, w_down, tables, expert_out)


def moe_expert_down_weighted(h, w_down, tables, expert_out=None):
    """Step 2b with the routing weight in the epilogue: expert_out row i =
    R(sorted_weight[i] * (h[i] W_down^T)); combine with moe_reduce_fused and
    no weights."""
    return _down(lib().moe_expert_down_weighted, h, w_down, tables, expert_out)


def forward_workspace(tables, H, D, dtype):
    """A workspace for moe_routed_forward and views of its h / expert_out."""
    code = _DTYPE_CODE[dtype]
    nbytes = lib().moe_forward_workspace_bytes(tables.T, tables.K, H, D, code)
    _require(nbytes > 0, MOE_ERR_SHAPE, "invalid workspace sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=tables.device)
    off = lib().moe_forward_workspace_expert_out_offset(tables.T, tables.K, H, D, code)
    P = tables.T * tables.K
    esz = torch.empty((), dtype=dtype).element_size()
    h = ws[:P * D * esz].view(dtype).view(P, D)
    eo = ws[off:off + P * H * esz].view(dtype).view(P, H)
    return ws, h, eo


def moe_routed_forward(x, w_gate, w_up, w_down, tables, y=None, workspace=None,
                       weighted_down=False):
    """Steps 2-3: y [T, H] of x.dtype. `workspace` from forward_workspace()
    (allocated here when None). weighted_down=True applies the routing
    weights in the down GEMM's epilogue and sums the rows unweighted
    (moe_routed_forward_weighted)."""
    _check_tensor(x, "x", None, 2, tables.device)
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_tensor(w, n, x.dtype, 3, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = forward_workspace(tables, H, D, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    fn = lib().moe_routed_forward_weighted if weighted_down else lib().moe_routed_forward
    check(fn(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), tables.ref, H, D,
             _DTYPE_CODE[x.dtype], _ptr(workspace), workspace.numel(), _ptr(y),
             _stream(x.device)))
    return y


FUSED_MAX_D_EXPERT = 2048   # MOE_FUSED_MAX_D_EXPERT of the C header


def moe_expert_fused(x, w_gate, w_up, w_down, tables, expert_out=None):
    """Steps 2a + 2b in one kernel for tables with block_m <= 32 (h of each
    row block stays in LDS): expert_out [T*K, H], bit-identical to
    moe_expert_down(moe_expert_gate_up(x))."""
    _check_tensor(x, "x", None, 2, tables.device)
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_tensor(w, n, x.dtype, 3, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    P = tables.T * tables.K
    if expert_out is None:
        expert_out = torch.empty(P, H, dtype=x.dtype, device=x.device)
    _check_tensor(expert_out, "expert_out", x.dtype, 2, tables.device)
    _require(tuple(expert_out.shape) == (P, H), MOE_ERR_SHAPE, "expert_out must be [T*K, H]")
    check(lib().moe_expert_fused(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), tables.ref, H,
                                 D, _DTYPE_CODE[x.dtype], _ptr(expert_out), _stream(x.device)))
    return expert_out


def fused_workspace(tables, H, dtype):
    """A workspace for moe_routed_forward_fused (expert_out only) and its
    expert_out view."""
    nbytes = lib().moe_fused_workspace_bytes(tables.T, tables.K, H, _DTYPE_CODE[dtype])
    _require(nbytes > 0, MOE_ERR_SHAPE, "invalid workspace sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=tables.device)
    P = tables.T * tables.K
    esz = torch.empty((), dtype=dtype).element_size()
    return ws, ws[:P * H * esz].view(dtype).view(P, H)


def moe_routed_forward_fused(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with the fused expert kernel (moe_routed_forward_fused):
    y [T, H], bit-identical to moe_routed_forward; `workspace` from
    fused_workspace() (allocated here when None)."""
    _check_tensor(x, "x", None, 2, tables.device)
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_tensor(w, n, x.dtype, 3, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = fused_workspace(tables, H, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_fused(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                         tables.ref, H, D, _DTYPE_CODE[x.dtype], _ptr(workspace),
                                         workspace.numel(), _ptr(y), _stream(x.device)))
    return y


NOALLOC_SCRATCH_BYTES = 80 << 20   # MOE_NOALLOC_SCRATCH_BYTES of the C header


def moe_routed_forward_noalloc(x, w_gate, w_up, w_down, tables, y):
    """Steps 2-3 with the library's static per-GPU scratch as the workspace
    (moe_routed_forward_noalloc: no device allocation anywhere in the call;
    y must be given). Calls that overlap on one GPU race on the scratch."""
    _check_tensor(x, "x", None, 2, tables.device)
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_tensor(w, n, x.dtype, 3, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_noalloc(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                           tables.ref, H, D, _DTYPE_CODE[x.dtype], _ptr(y),
                                           _stream(x.device)))
    return y


def moe_routed_forward_weighted(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with the weighted down epilogue and an unweighted combine."""
    return moe_routed_forward(x, w_gate, w_up, w_down, tables, y, workspace, True)


class FP8Weights:
    """Stacked expert weights in FP8 E4M3: `codes` uint8 [E, N, Kd] and one
    fp32 scale per row, `scales` [E, N] (value = scale * decoded code)."""

    def __init__(self, codes, scales):
        _check_tensor(codes, "codes", torch.uint8, 3)
        _check_tensor(scales, "scales", torch.float32, 2, codes.device)
        _require(tuple(scales.shape) == tuple(codes.shape[:2]), MOE_ERR_SHAPE,
                 "scales must be [E, N] = %s" % (tuple(codes.shape[:2]),))
        self.codes = codes
        self.scales = scales

    @property
    def shape(self):
        return self.codes.shape

    def dim(self):
        return 3


def quantize_fp8_rows(w):
    """moe_quantize_fp8_rows on stacked weights w [E, N, Kd] (fp16 / bf16 /
    fp32): per-row scale amax / 448 and E4M3 codes. Returns FP8Weights."""
    _check_tensor(w, "w", None, 3)
    _require(w.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "w must be float16, bfloat16 or float32")
    E, N, Kd = w.shape
    codes = torch.empty((E, N, Kd), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, N), dtype=torch.float32, device=w.device)
    check(lib().moe_quantize_fp8_rows(_ptr(w), E * N, Kd, _DTYPE_CODE[w.dtype], _ptr(codes),
                                      _ptr(scales), _stream(w.device)))
    return FP8Weights(codes, scales)


def _check_w8(w, name, device):
    _require(isinstance(w, FP8Weights), MOE_ERR_DTYPE, "%s must be FP8Weights" % name)
    _require(w.codes.device == device, MOE_ERR_SHAPE, "%s is on another device" % name)


def moe_expert_gate_up_w8(x, w_gate, w_up, tables, h=None):
    """Step 2a with FP8 weights (FP8Weights [E, D, H]); x and h 16-bit."""
    _check_tensor(x, "x", None, 2, tables.device)
    _require(x.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "FP8 weights take float16 or bfloat16 activations")
    for n, w in (("w_gate", w_gate), ("w_up", w_up)):
        _check_w8(w, n, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, None, tables, True)
    if h is None:
        h = torch.empty(tables.T * tables.K, D, dtype=x.dtype, device=x.device)
    _check_tensor(h, "h", x.dtype, 2, tables.device)
    check(lib().moe_expert_gate_up_w8(_ptr(x), _ptr(w_gate.codes), _ptr(w_up.codes),
                                      _ptr(w_gate.scales), _ptr(w_up.scales), tables.ref, H, D,
                                      _DTYPE_CODE[x.dtype], _ptr(h), _stream(x.device)))
    return h


def moe_expert_down_w8(h, w_down, tables, expert_out=None):
    """Step 2b with FP8 weights (FP8Weights [E, H, D]); h and expert_out 16-bit."""
    _check_tensor(h, "h", None, 2, tables.device)
    _require(h.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "FP8 weights take float16 or bfloat16 activations")
    _check_w8(w_down, "w_down", tables.device)
    H, D = _expert_shapes(h, w_down, None, None, tables, False)
    if expert_out is None:
        expert_out = torch.empty(tables.T * tables.K, H, dtype=h.dtype, device=h.device)
    _check_tensor(expert_out, "expert_out", h.dtype, 2, tables.device)
    check(lib().moe_expert_down_w8(_ptr(h), _ptr(w_down.codes), _ptr(w_down.scales), tables.ref,
                                   H, D, _DTYPE_CODE[h.dtype], _ptr(expert_out),
                                   _stream(h.device)))
    return expert_out


def moe_routed_forward_w8(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with FP8 weights: y [T, H] of x.dtype."""
    _check_tensor(x, "x", None, 2, tables.device)
    _require(x.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "FP8 weights take float16 or bfloat16 activations")
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_w8(w, n, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = forward_workspace(tables, H, D, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_w8(_ptr(x), _ptr(w_gate.codes), _ptr(w_up.codes),
                                      _ptr(w_down.codes), _ptr(w_gate.scales),
                                      _ptr(w_up.scales), _ptr(w_down.scales), tables.ref, H, D,
                                      _DTYPE_CODE[x.dtype], _ptr(workspace), workspace.numel(),
                                      _ptr(y), _stream(x.device)))
    return y


def quantize_fp8_act_rows(a, q=None, scales=None):
    """moe_quantize_fp8_rows on activations a [rows, cols] (fp16 / bf16 /
    fp32): E4M3 codes (uint8) and fp32 scales amax / 448 per row. Returns
    (q, scales) (written into q / scales when given)."""
    _check_tensor(a, "a", None, 2)
    _require(a.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "a must be float16, bfloat16 or float32")
    rows, cols = a.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=a.device)
    _check_tensor(q, "q", torch.uint8, 2, a.device)
    _check_tensor(scales, "scales", torch.float32, 1, a.device)
    _require(tuple(q.shape) == (rows, cols) and scales.numel() == rows, MOE_ERR_SHAPE,
             "q must be [rows, cols] and scales [rows]")
    check(lib().moe_quantize_fp8_rows(_ptr(a), rows, cols, _DTYPE_CODE[a.dtype], _ptr(q),
                                      _ptr(scales), _stream(a.device)))
    return q, scales


def _check_w8a8_act(q, s, name, rows, cols, device):
    _check_tensor(q, name, torch.uint8, 2, device)
    _check_tensor(s, name + " scales", torch.float32, 1, device)
    _require(tuple(q.shape) == (rows, cols) and s.numel() == rows, MOE_ERR_SHAPE,
             "%s must be [%d, %d] with %d scales" % (name, rows, cols, rows))


def moe_expert_gate_up_w8a8(xq, sx, w_gate, w_up, tables, dtype=torch.bfloat16, h=None):
    """Step 2a with W8A8 experts: E4M3 activations xq [T, H] with per-token
    scales sx [T] against FP8Weights [E, D, H]; h [P, D] of dtype."""
    for n, w in (("w_gate", w_gate), ("w_up", w_up)):
        _check_w8(w, n, tables.device)
    E, D, H = w_gate.shape
    _check_w8a8_act(xq, sx, "xq", tables.T, H, tables.device)
    _require(tuple(w_up.shape) == (E, D, H) and E == tables.E, MOE_ERR_SHAPE,
             "w_gate and w_up must be [E, D, H]")
    _require(dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE, "dtype must be 16-bit")
    if h is None:
        h = torch.empty(tables.T * tables.K, D, dtype=dtype, device=xq.device)
    _check_tensor(h, "h", dtype, 2, tables.device)
    check(lib().moe_expert_gate_up_w8a8(_ptr(xq), _ptr(sx), _ptr(w_gate.codes), _ptr(w_up.codes),
                                        _ptr(w_gate.scales), _ptr(w_up.scales), tables.ref, H, D,
                                        _DTYPE_CODE[dtype], _ptr(h), _stream(xq.device)))
    return h


def moe_expert_down_w8a8(hq, sh, w_down, tables, dtype=torch.bfloat16, expert_out=None):
    """Step 2b with W8A8 experts: E4M3 rows hq [P, D] with per-row scales
    sh [P] against FP8Weights [E, H, D]; expert_out [P, H] of dtype."""
    _check_w8(w_down, "w_down", tables.device)
    E, H, D = w_down.shape
    _require(E == tables.E, MOE_ERR_SHAPE, "w_down must be [E, H, D]")
    _check_w8a8_act(hq, sh, "hq", tables.T * tables.K, D, tables.device)
    _require(dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE, "dtype must be 16-bit")
    if expert_out is None:
        expert_out = torch.empty(tables.T * tables.K, H, dtype=dtype, device=hq.device)
    _check_tensor(expert_out, "expert_out", dtype, 2, tables.device)
    check(lib().moe_expert_down_w8a8(_ptr(hq), _ptr(sh), _ptr(w_down.codes), _ptr(w_down.scales),
                                     tables.ref, H, D, _DTYPE_CODE[dtype], _ptr(expert_out),
                                     _stream(hq.device)))
    return expert_out


def forward_w8a8_workspace(tables, H, D, dtype):
    """A workspace for moe_routed_forward_w8a8 and views of its buffers:
    (ws, h, expert_out, xq, sx, hq, sh)."""
    code = _DTYPE_CODE[dtype]
    nbytes = lib().moe_forward_w8a8_workspace_bytes(tables.T, tables.K, H, D, code)
    _require(nbytes > 0, MOE_ERR_SHAPE, "invalid workspace sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=tables.device)
    base = lib().moe_forward_workspace_bytes(tables.T, tables.K, H, D, code)
    off = lib().moe_forward_workspace_expert_out_offset(tables.T, tables.K, H, D, code)
    T, P = tables.T, tables.T * tables.K
    esz = torch.empty((), dtype=dtype).element_size()
    up = lambda v: (v + 255) // 256 * 256
    h = ws[:P * D * esz].view(dtype).view(P, D)
    eo = ws[off:off + P * H * esz].view(dtype).view(P, H)
    o_xq = base
    o_sx = o_xq + up(T * H)
    o_hq = o_sx + up(T * 4)
    o_sh = o_hq + up(P * D)
    xq = ws[o_xq:o_xq + T * H].view(T, H)
    sx = ws[o_sx:o_sx + T * 4].view(torch.float32)
    hq = ws[o_hq:o_hq + P * D].view(P, D)
    sh = ws[o_sh:o_sh + P * 4].view(torch.float32)
    return ws, h, eo, xq, sx, hq, sh


def moe_routed_forward_w8a8(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with W8A8 experts (FP8Weights; x 16-bit, quantised to E4M3
    per token inside, h per sorted row): y [T, H] of x.dtype."""
    _check_tensor(x, "x", None, 2, tables.device)
    _require(x.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "W8A8 experts take float16 or bfloat16 activations")
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_w8(w, n, tables.device)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = forward_w8a8_workspace(tables, H, D, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_w8a8(_ptr(x), _ptr(w_gate.codes), _ptr(w_up.codes),
                                        _ptr(w_down.codes), _ptr(w_gate.scales),
                                        _ptr(w_up.scales), _ptr(w_down.scales), tables.ref, H, D,
                                        _DTYPE_CODE[x.dtype], _ptr(workspace), workspace.numel(),
                                        _ptr(y), _stream(x.device)))
    return y


class W4Weights:
    """Stacked expert weights in int4: `packed` uint8 [E, N, Kd/2] (field 2i
    in the low nibble of byte i) and one fp32 scale per row, `scales` [E, N]
    (value = scale * field). `shape` is the logical [E, N, Kd]."""

    def __init__(self, packed, scales):
        _check_tensor(packed, "packed", torch.uint8, 3)
        _check_tensor(scales, "scales", torch.float32, 2, packed.device)
        _require(tuple(scales.shape) == tuple(packed.shape[:2]), MOE_ERR_SHAPE,
                 "scales must be [E, N] = %s" % (tuple(packed.shape[:2]),))
        self.packed = packed
        self.scales = scales

    @property
    def shape(self):
        E, N, half = self.packed.shape
        return torch.Size((E, N, 2 * half))

    def dim(self):
        return 3


def quantize_int8_rows(a, q=None, scales=None):
    """moe_quantize_int8_rows on a [rows, cols] (fp16 / bf16 / fp32): int8
    codes in [-127, 127] and fp32 scales amax / 127. Returns (q, scales)
    (written into q / scales when given)."""
    _check_tensor(a, "a", None, 2)
    _require(a.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "a must be float16, bfloat16 or float32")
    rows, cols = a.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=a.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=a.device)
    _check_tensor(q, "q", torch.int8, 2, a.device)
    _check_tensor(scales, "scales", torch.float32, 1, a.device)
    _require(tuple(q.shape) == (rows, cols) and scales.shape[0] == rows, MOE_ERR_SHAPE,
             "q must be [%d, %d] and scales [%d]" % (rows, cols, rows))
    check(lib().moe_quantize_int8_rows(_ptr(a), rows, cols, _DTYPE_CODE[a.dtype], _ptr(q),
                                       _ptr(scales), _stream(a.device)))
    return q, scales


def quantize_int4_rows(w):
    """moe_quantize_int4_rows on stacked weights w [E, N, Kd] (Kd even):
    per-row scale amax / 7 and int4 codes in [-8, 7], packed. Returns
    W4Weights."""
    _check_tensor(w, "w", None, 3)
    _require(w.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "w must be float16, bfloat16 or float32")
    E, N, Kd = w.shape
    _require(Kd % 2 == 0, MOE_ERR_SHAPE, "the row length must be even")
    packed = torch.empty((E, N, Kd // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, N), dtype=torch.float32, device=w.device)
    check(lib().moe_quantize_int4_rows(_ptr(w), E * N, Kd, _DTYPE_CODE[w.dtype], _ptr(packed),
                                       _ptr(scales), _stream(w.device)))
    return W4Weights(packed, scales)


def w4a8_gemm(A, B, Ct=None):
    """moe_w4a8_gemm: Ct [N, M] int32 = sum_k A[m, k] * B4[n, k] for A int8
    [M, K] and packed int4 B uint8 [N, K/2]."""
    _check_tensor(A, "A", torch.int8, 2)
    _check_tensor(B, "B", torch.uint8, 2, A.device)
    M, K = A.shape
    N = B.shape[0]
    _require(B.shape[1] * 2 == K, MOE_ERR_SHAPE, "B must be [N, K/2] (got %s)" % (tuple(B.shape),))
    if Ct is None:
        Ct = torch.empty((N, M), dtype=torch.int32, device=A.device)
    _check_tensor(Ct, "Ct", torch.int32, 2, A.device)
    _require(tuple(Ct.shape) == (N, M), MOE_ERR_SHAPE, "Ct must be [N, M]")
    check(lib().moe_w4a8_gemm(_ptr(A), _ptr(B), M, N, K, _ptr(Ct), _stream(A.device)))
    return Ct


def _w4_shapes(act, scales, w_a, w_b, w_down, tables, gate_up, dtype):
    _require(dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "W4A8 experts produce float16 or bfloat16")
    _check_tensor(act, "activations", torch.int8, 2, tables.device)
    _check_tensor(scales, "activation scales", torch.float32, 1, tables.device)
    for n, w in (("w_a", w_a), ("w_b", w_b), ("w_down", w_down)):
        if w is not None:
            _require(isinstance(w, W4Weights), MOE_ERR_DTYPE, "%s must be W4Weights" % n)
            _require(w.packed.device == tables.device, MOE_ERR_SHAPE, "%s is on another device" % n)
    E = tables.E
    rows, kd = act.shape
    _require(scales.shape[0] == rows, MOE_ERR_SHAPE, "one activation scale per row")
    if gate_up:
        _require(rows == tables.T, MOE_ERR_SHAPE, "xq has %d rows, tables %d tokens" % (rows, tables.T))
        H = kd
        _require(w_a.shape[0] == E and w_a.shape[2] == H, MOE_ERR_SHAPE,
                 "w_gate must be [E=%d, D, H=%d] (got %s)" % (E, H, tuple(w_a.shape)))
        D = w_a.shape[1]
        _require(tuple(w_b.shape) == (E, D, H), MOE_ERR_SHAPE, "w_up must be [%d, %d, %d]" % (E, D, H))
        if w_down is not None:
            _require(tuple(w_down.shape) == (E, H, D), MOE_ERR_SHAPE,
                     "w_down must be [%d, %d, %d]" % (E, H, D))
        return H, D
    _require(rows == tables.T * tables.K, MOE_ERR_SHAPE, "hq must have T*K rows")
    D = kd
    _require(w_a.shape[0] == E and w_a.shape[2] == D, MOE_ERR_SHAPE,
             "w_down must be [E=%d, H, D=%d] (got %s)" % (E, D, tuple(w_a.shape)))
    return w_a.shape[1], D


def moe_expert_gate_up_w4a8(xq, sx, w_gate, w_up, tables, dtype=torch.bfloat16, h=None):
    """Step 2a with W4A8 experts: xq int8 [T, H] with scales sx [T] against
    W4Weights [E, D, H]; h [T*K, D] of dtype."""
    H, D = _w4_shapes(xq, sx, w_gate, w_up, None, tables, True, dtype)
    if h is None:
        h = torch.empty(tables.T * tables.K, D, dtype=dtype, device=xq.device)
    _check_tensor(h, "h", dtype, 2, tables.device)
    check(lib().moe_expert_gate_up_w4a8(_ptr(xq), _ptr(sx), _ptr(w_gate.packed), _ptr(w_up.packed),
                                        _ptr(w_gate.scales), _ptr(w_up.scales), tables.ref, H, D,
                                        _DTYPE_CODE[dtype], _ptr(h), _stream(xq.device)))
    return h


def moe_expert_down_w4a8(hq, sh, w_down, tables, dtype=torch.bfloat16, expert_out=None):
    """Step 2b with W4A8 experts: hq int8 [T*K, D] with scales sh [T*K]
    against W4Weights [E, H, D]; expert_out [T*K, H] of dtype."""
    H, D = _w4_shapes(hq, sh, w_down, None, None, tables, False, dtype)
    if expert_out is None:
        expert_out = torch.empty(tables.T * tables.K, H, dtype=dtype, device=hq.device)
    _check_tensor(expert_out, "expert_out", dtype, 2, tables.device)
    check(lib().moe_expert_down_w4a8(_ptr(hq), _ptr(sh), _ptr(w_down.packed), _ptr(w_down.scales),
                                     tables.ref, H, D, _DTYPE_CODE[dtype], _ptr(expert_out),
                                     _stream(hq.device)))
    return expert_out


def forward_w4a8_workspace(tables, H, D, dtype):
    """A workspace for moe_routed_forward_w4a8 and views of its buffers:
    (ws, h, expert_out, xq, sx, hq, sh)."""
    code = _DTYPE_CODE[dtype]
    nbytes = lib().moe_forward_w4a8_workspace_bytes(tables.T, tables.K, H, D, code)
    _require(nbytes > 0, MOE_ERR_SHAPE, "invalid workspace sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=tables.device)
    base = lib().moe_forward_workspace_bytes(tables.T, tables.K, H, D, code)
    off = lib().moe_forward_workspace_expert_out_offset(tables.T, tables.K, H, D, code)
    T, P = tables.T, tables.T * tables.K
    esz = torch.empty((), dtype=dtype).element_size()
    up = lambda v: (v + 255) // 256 * 256
    h = ws[:P * D * esz].view(dtype).view(P, D)
    eo = ws[off:off + P * H * esz].view(dtype).view(P, H)
    o_xq = base
    o_sx = o_xq + up(T * H)
    o_hq = o_sx + up(T * 4)
    o_sh = o_hq + up(P * D)
    xq = ws[o_xq:o_xq + T * H].view(torch.int8).view(T, H)
    sx = ws[o_sx:o_sx + T * 4].view(torch.float32)
    hq = ws[o_hq:o_hq + P * D].view(torch.int8).view(P, D)
    sh = ws[o_sh:o_sh + P * 4].view(torch.float32)
    return ws, h, eo, xq, sx, hq, sh


def moe_routed_forward_w4a8(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with W4A8 experts (W4Weights; x 16-bit, quantised to int8
    per token inside): y [T, H] of x.dtype."""
    _check_tensor(x, "x", None, 2, tables.device)
    _require(x.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "W4A8 experts take float16 or bfloat16 activations")
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _require(isinstance(w, W4Weights), MOE_ERR_DTYPE, "%s must be W4Weights" % n)
        _require(w.packed.device == tables.device, MOE_ERR_SHAPE, "%s is on another device" % n)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = forward_w4a8_workspace(tables, H, D, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_w4a8(_ptr(x), _ptr(w_gate.packed), _ptr(w_up.packed),
                                        _ptr(w_down.packed), _ptr(w_gate.scales),
                                        _ptr(w_up.scales), _ptr(w_down.scales), tables.ref, H, D,
                                        _DTYPE_CODE[x.dtype], _ptr(workspace), workspace.numel(),
                                        _ptr(y), _stream(x.device)))
    return y


class MXWeights:
    """Stacked expert weights in MXFP4: `packed` uint8 [E, N, Kd/2] (E2M1
    codes, element 2i in the low nibble) and E8M0 block scales `scales`
    uint8 [E, N, Kd/32]. `shape` is the logical [E, N, Kd]."""

    def __init__(self, packed, scales):
        _check_tensor(packed, "packed", torch.uint8, 3)
        _check_tensor(scales, "scales", torch.uint8, 3, packed.device)
        E, N, half = packed.shape
        _require(tuple(scales.shape) == (E, N, half * 2 // 32), MOE_ERR_SHAPE,
                 "scales must be [E, N, Kd/32] = %s" % ((E, N, half * 2 // 32),))
        self.packed = packed
        self.scales = scales

    @property
    def shape(self):
        E, N, half = self.packed.shape
        return torch.Size((E, N, 2 * half))

    def dim(self):
        return 3


def quantize_mx_rows(v, fmt=MX_FP8, codes=None, scales=None):
    """moe_quantize_mx_rows on v [rows, cols] (fp16 / bf16 / fp32, cols a
    multiple of 32): MX codes (MX_FP8: [rows, cols]; MX_FP4: packed [rows,
    cols/2]) and E8M0 scales [rows, cols/32]. Returns (codes, scales)."""
    _check_tensor(v, "v", None, 2)
    _require(v.dtype in _DTYPE_CODE, MOE_ERR_DTYPE, "v must be float16, bfloat16 or float32")
    rows, cols = v.shape
    cshape = (rows, cols) if fmt == MX_FP8 else (rows, cols // 2)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=v.device)
    _check_tensor(codes, "codes", torch.uint8, 2, v.device)
    _check_tensor(scales, "scales", torch.uint8, 2, v.device)
    _require(tuple(codes.shape) == cshape and tuple(scales.shape) == (rows, cols // 32),
             MOE_ERR_SHAPE, "codes must be %s and scales [%d, %d]" % (cshape, rows, cols // 32))
    check(lib().moe_quantize_mx_rows(_ptr(v), rows, cols, _DTYPE_CODE[v.dtype], fmt, _ptr(codes),
                                      _ptr(scales), _stream(v.device)))
    return codes, scales


def quantize_mx_weights(w):
    """MXFP4 quantisation of stacked weights w [E, N, Kd]. Returns MXWeights."""
    _check_tensor(w, "w", None, 3)
    E, N, Kd = w.shape
    codes, scales = quantize_mx_rows(w.view(E * N, Kd), MX_FP4)
    return MXWeights(codes.view(E, N, Kd // 2), scales.view(E, N, Kd // 32))


def _mx_shapes(act, scales, w_a, w_b, w_down, tables, gate_up, dtype):
    _require(dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "MX experts produce float16 or bfloat16")
    _check_tensor(act, "activations", torch.uint8, 2, tables.device)
    _check_tensor(scales, "activation scales", torch.uint8, 2, tables.device)
    for n, w in (("w_a", w_a), ("w_b", w_b), ("w_down", w_down)):
        if w is not None:
            _require(isinstance(w, MXWeights), MOE_ERR_DTYPE, "%s must be MXWeights" % n)
            _require(w.packed.device == tables.device, MOE_ERR_SHAPE, "%s is on another device" % n)
    E = tables.E
    rows, kd = act.shape
    _require(tuple(scales.shape) == (rows, kd // 32), MOE_ERR_SHAPE, "activation scales must be [rows, kd/32]")
    if gate_up:
        _require(rows == tables.T, MOE_ERR_SHAPE, "xq has %d rows, tables %d tokens" % (rows, tables.T))
        H = kd
        _require(w_a.shape[0] == E and w_a.shape[2] == H, MOE_ERR_SHAPE,
                 "w_gate must be [E=%d, D, H=%d] (got %s)" % (E, H, tuple(w_a.shape)))
        D = w_a.shape[1]
        _require(tuple(w_b.shape) == (E, D, H), MOE_ERR_SHAPE, "w_up must be [%d, %d, %d]" % (E, D, H))
        return H, D
    _require(rows == tables.T * tables.K, MOE_ERR_SHAPE, "hq must have T*K rows")
    D = kd
    _require(w_a.shape[0] == E and w_a.shape[2] == D, MOE_ERR_SHAPE,
             "w_down must be [E=%d, H, D=%d] (got %s)" % (E, D, tuple(w_a.shape)))
    return w_a.shape[1], D


def moe_expert_gate_up_mx(xq, xs, w_gate, w_up, tables, dtype=torch.bfloat16, h=None):
    """Step 2a with MX experts: MXFP8 xq [T, H] (scales xs [T, H/32])
    against MXWeights [E, D, H]; h [T*K, D] of dtype."""
    H, D = _mx_shapes(xq, xs, w_gate, w_up, None, tables, True, dtype)
    if h is None:
        h = torch.empty(tables.T * tables.K, D, dtype=dtype, device=xq.device)
    _check_tensor(h, "h", dtype, 2, tables.device)
    check(lib().moe_expert_gate_up_mx(_ptr(xq), _ptr(xs), _ptr(w_gate.packed), _ptr(w_up.packed),
                                      _ptr(w_gate.scales), _ptr(w_up.scales), tables.ref, H, D,
                                      _DTYPE_CODE[dtype], _ptr(h), _stream(xq.device)))
    return h


def moe_expert_down_mx(hq, hs, w_down, tables, dtype=torch.bfloat16, expert_out=None):
    """Step 2b with MX experts: MXFP8 hq [T*K, D] (scales hs [T*K, D/32])
    against MXWeights [E, H, D]; expert_out [T*K, H] of dtype."""
    H, D = _mx_shapes(hq, hs, w_down, None, None, tables, False, dtype)
    if expert_out is None:
        expert_out = torch.empty(tables.T * tables.K, H, dtype=dtype, device=hq.device)
    _check_tensor(expert_out, "expert_out", dtype, 2, tables.device)
    check(lib().moe_expert_down_mx(_ptr(hq), _ptr(hs), _ptr(w_down.packed), _ptr(w_down.scales),
                                   tables.ref, H, D, _DTYPE_CODE[dtype], _ptr(expert_out),
                                   _stream(hq.device)))
    return expert_out


def forward_mx_workspace(tables, H, D, dtype):
    """A workspace for moe_routed_forward_mx and views of its buffers:
    (ws, h, expert_out, xq, xs, hq, hs)."""
    code = _DTYPE_CODE[dtype]
    nbytes = lib().moe_forward_mx_workspace_bytes(tables.T, tables.K, H, D, code)
    _require(nbytes > 0, MOE_ERR_SHAPE, "invalid workspace sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=tables.device)
    base = lib().moe_forward_workspace_bytes(tables.T, tables.K, H, D, code)
    off = lib().moe_forward_workspace_expert_out_offset(tables.T, tables.K, H, D, code)
    T, P = tables.T, tables.T * tables.K
    esz = torch.empty((), dtype=dtype).element_size()
    up = lambda v: (v + 255) // 256 * 256
    h = ws[:P * D * esz].view(dtype).view(P, D)
    eo = ws[off:off + P * H * esz].view(dtype).view(P, H)
    o_xq = base
    o_xs = o_xq + up(T * H)
    o_hq = o_xs + up(T * (H // 32))
    o_hs = o_hq + up(P * D)
    xq = ws[o_xq:o_xq + T * H].view(T, H)
    xs = ws[o_xs:o_xs + T * (H // 32)].view(T, H // 32)
    hq = ws[o_hq:o_hq + P * D].view(P, D)
    hs = ws[o_hs:o_hs + P * (D // 32)].view(P, D // 32)
    return ws, h, eo, xq, xs, hq, hs


def moe_routed_forward_mx(x, w_gate, w_up, w_down, tables, y=None, workspace=None):
    """Steps 2-3 with MX experts (MXWeights; x 16-bit, quantised to MXFP8
    per token inside): y [T, H] of x.dtype."""
    _check_tensor(x, "x", None, 2, tables.device)
    _require(x.dtype in (torch.float16, torch.bfloat16), MOE_ERR_DTYPE,
             "MX experts take float16 or bfloat16 activations")
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _require(isinstance(w, MXWeights), MOE_ERR_DTYPE, "%s must be MXWeights" % n)
        _require(w.packed.device == tables.device, MOE_ERR_SHAPE, "%s is on another device" % n)
    H, D = _expert_shapes(x, w_gate, w_up, w_down, tables, True)
    if workspace is None:
        workspace = forward_mx_workspace(tables, H, D, x.dtype)[0]
    _check_tensor(workspace, "workspace", torch.uint8, 1, tables.device)
    if y is None:
        y = torch.empty(tables.T, H, dtype=x.dtype, device=x.device)
    _check_tensor(y, "y", x.dtype, 2, tables.device)
    _require(tuple(y.shape) == (tables.T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    check(lib().moe_routed_forward_mx(_ptr(x), _ptr(w_gate.packed), _ptr(w_up.packed),
                                      _ptr(w_down.packed), _ptr(w_gate.scales),
                                      _ptr(w_up.scales), _ptr(w_down.scales), tables.ref, H, D,
                                      _DTYPE_CODE[x.dtype], _ptr(workspace), workspace.numel(),
                                      _ptr(y), _stream(x.device)))
    return y


def moe_reduce_fused(expert_out, token_topk_to_pos, topk_weights=None, out_dtype=None, y=None,
                     x_sf=None, sf=None):
    """Step 3: y[t] = sf[t] * sum_k (w[t,k] * x_sf[pos[t,k]]) * expert_out[pos[t,k]]
    over pos >= 0, fp32 accumulation, one cast to out_dtype (default:
    expert_out's dtype). topk_weights, x_sf (fp32 [rows]) and sf (fp32 [T])
    are optional (None = ones). expert_out and y may be float16, bfloat16,
    float32 or float8_e4m3fn."""
    _check_tensor(expert_out, "expert_out", None, 2)
    _require(expert_out.dtype in _REDUCE_CODE, MOE_ERR_DTYPE,
             "expert_out dtype %s not supported" % expert_out.dtype)
    dev = expert_out.device
    _check_tensor(token_topk_to_pos, "token_topk_to_pos", torch.int32, 2, dev)
    T, K = token_topk_to_pos.shape
    R, H = expert_out.shape
    if topk_weights is not None:
        _check_tensor(topk_weights, "topk_weights", torch.float32, 2, dev)
        _require(tuple(topk_weights.shape) == (T, K), MOE_ERR_SHAPE,
                 "topk_weights shape %s != token_topk_to_pos shape %s"
                 % (tuple(topk_weights.shape), (T, K)))
    if x_sf is not None:
        _check_tensor(x_sf, "x_sf", torch.float32, 1, dev)
        _require(x_sf.shape[0] == R, MOE_ERR_SHAPE, "x_sf must hold one scale per expert_out row")
    if sf is not None:
        _check_tensor(sf, "sf", torch.float32, 1, dev)
        _require(sf.shape[0] == T, MOE_ERR_SHAPE, "sf must hold one scale per token")
    out_dtype = expert_out.dtype if out_dtype is None else out_dtype
    _require(out_dtype in _REDUCE_CODE, MOE_ERR_DTYPE, "out_dtype %s not supported" % out_dtype)
    if y is None:
        y = torch.empty(T, H, dtype=out_dtype, device=dev)
    _check_tensor(y, "y", out_dtype, 2, dev)
    _require(tuple(y.shape) == (T, H), MOE_ERR_SHAPE, "y must be [T, H]")
    if x_sf is None and sf is None:
        check(lib().moe_reduce_fused(_ptr(expert_out), R, _ptr(token_topk_to_pos),
                                     _ptr(topk_weights), T, K, H, _REDUCE_CODE[expert_out.dtype],
                                     _REDUCE_CODE[out_dtype], _ptr(y), _stream(dev)))
    else:
        check(lib().moe_reduce_fused_scaled(_ptr(expert_out), R, _ptr(token_topk_to_pos),
                                            _ptr(topk_weights), _ptr(x_sf), _ptr(sf), T, K, H,
                                            _REDUCE_CODE[expert_out.dtype],
                                            _REDUCE_CODE[out_dtype], _ptr(y), _stream(dev)))
    return y
