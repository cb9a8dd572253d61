"""ctypes view of libmoe_routed.so (the C ABI declared in include/moe_routed.h).

Loads the in-tree library and fails loudly if it has not been built: there is
no fallback implementation of any step.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_routed.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE = 0, 1, 2, 3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 4, 5, 6
MOE_F16, MOE_BF16, MOE_F32, MOE_FP8_E4M3 = 0, 1, 2, 3


class MoeTablesStruct(ctypes.Structure):
    """Mirror of `struct moe_tables` (field order and types as in the header)."""
    _fields_ = [
        ("T", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
        ("block_m", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("num_chunks", ctypes.c_int32),
        ("group_sizes", ctypes.c_void_p), ("group_offsets", ctypes.c_void_p),
        ("group_padded_offsets", ctypes.c_void_p), ("block_expert", ctypes.c_void_p),
        ("sorted_pair", ctypes.c_void_p), ("sorted_token", ctypes.c_void_p),
        ("sorted_weight", ctypes.c_void_p), ("token_topk_to_pos", ctypes.c_void_p),
        ("topk_weights", ctypes.c_void_p), ("status", ctypes.c_void_p),
        ("active_blocks", ctypes.c_void_p), ("active_count", ctypes.c_void_p),
        ("chunk_counts", ctypes.c_void_p), ("chunk_flags", ctypes.c_void_p),
        ("pair_rank", ctypes.c_void_p),
    ]


class MoeError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__("%s: %s" % (status_string(status), message))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmoe_routed.so is not built (expected at %s); run "
                "__graft_entry__.build() or python mixture_experts_routed_moe_amd/build.py"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
        tp = ctypes.POINTER(MoeTablesStruct)
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_tables_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_tables_bytes.restype = sz
        L.moe_tables_bind.argtypes = [tp, vp, sz, i32, i32, i32, i32]
        L.moe_tables_bind.restype = i32
        L.moe_dispatch.argtypes = [vp, vp, tp, vp]
        L.moe_dispatch.restype = i32
        L.moe_expert_gate_up.argtypes = [vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_gate_up.restype = i32
        L.moe_expert_down.argtypes = [vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down.restype = i32
        L.moe_forward_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.moe_forward_workspace_bytes.restype = sz
        L.moe_forward_workspace_expert_out_offset.argtypes = [i32, i32, i32, i32, i32]
        L.moe_forward_workspace_expert_out_offset.restype = sz
        L.moe_routed_forward.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, sz, vp, vp]
        L.moe_routed_forward.restype = i32
        L.moe_routed_forward_noalloc.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_routed_forward_noalloc.restype = i32
        L.moe_expert_fused.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_fused.restype = i32
        L.moe_fused_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_fused_workspace_bytes.restype = sz
        L.moe_routed_forward_fused.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, sz, vp, vp]
        L.moe_routed_forward_fused.restype = i32
        L.moe_expert_down_weighted.argtypes = [vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down_weighted.restype = i32
        L.moe_routed_forward_weighted.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, sz, vp,
                                                  vp]
        L.moe_routed_forward_weighted.restype = i32
        L.moe_reduce_fused.argtypes = [vp, i64, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.moe_reduce_fused.restype = i32
        L.moe_quantize_fp8_rows.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.moe_quantize_fp8_rows.restype = i32
        L.moe_expert_gate_up_w8.argtypes = [vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_gate_up_w8.restype = i32
        L.moe_expert_down_w8.argtypes = [vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down_w8.restype = i32
        L.moe_routed_forward_w8.argtypes = [vp, vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, sz,
                                            vp, vp]
        L.moe_routed_forward_w8.restype = i32
        L.moe_gate.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.moe_gate.restype = i32
        L.moe_reduce_fused_scaled.argtypes = [vp, i64, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                              vp, vp]
        L.moe_reduce_fused_scaled.restype = i32
        L.moe_quantize_int8_rows.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.moe_quantize_int8_rows.restype = i32
        L.moe_quantize_int4_rows.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.moe_quantize_int4_rows.restype = i32
        L.moe_w4a8_gemm.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.moe_w4a8_gemm.restype = i32
        L.moe_expert_gate_up_w4a8.argtypes = [vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_gate_up_w4a8.restype = i32
        L.moe_expert_down_w4a8.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down_w4a8.restype = i32
        L.moe_expert_gate_up_w8a8.argtypes = [vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_gate_up_w8a8.restype = i32
        L.moe_expert_down_w8a8.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down_w8a8.restype = i32
        L.moe_forward_w8a8_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.moe_forward_w8a8_workspace_bytes.restype = sz
        L.moe_routed_forward_w8a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp,
                                              sz, vp, vp]
        L.moe_routed_forward_w8a8.restype = i32
        L.moe_forward_w4a8_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.moe_forward_w4a8_workspace_bytes.restype = sz
        L.moe_routed_forward_w4a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp,
                                              sz, vp, vp]
        L.moe_routed_forward_w4a8.restype = i32
        L.moe_quantize_mx_rows.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
        L.moe_quantize_mx_rows.restype = i32
        L.moe_expert_gate_up_mx.argtypes = [vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_gate_up_mx.restype = i32
        L.moe_expert_down_mx.argtypes = [vp, vp, vp, vp, tp, i32, i32, i32, vp, vp]
        L.moe_expert_down_mx.restype = i32
        L.moe_forward_mx_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.moe_forward_mx_workspace_bytes.restype = sz
        L.moe_routed_forward_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, tp, i32, i32, i32, vp, sz,
                                            vp, vp]
        L.moe_routed_forward_mx.restype = i32
        _lib = L
    return _lib


def status_string(status):
    return lib().moe_status_string(status).decode()


def check(status):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())
