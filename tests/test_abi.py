"""The C ABI without a GPU: the library loads, exports every function the
headers declare, and its host-side validation rejects bad arguments before
touching the device (only calls that fail validation are made here)."""
import ctypes
import glob
import os
import re

import pytest

import mixture_experts_routed_moe_amd as mr
from mixture_experts_routed_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_three_calls():
    names = _declared_functions()
    assert {"moe_dispatch", "moe_routed_forward", "moe_reduce_fused"} <= names
    assert len(names) >= 10


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in sorted(_declared_functions()) if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    L = _lib.lib()
    assert [L.moe_status_string(i).decode() for i in range(7)] == [
        "MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_DTYPE", "MOE_ERR_UNSUPPORTED",
        "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]


def test_struct_matches_header_field_count():
    text = open(os.path.join(ROOT, "include", "moe_routed.h")).read()
    body = re.search(r"typedef struct moe_tables \{(.*?)\} moe_tables;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\*?\s*(\w+)\s*[,;]", body)
    assert [f for f, _ in _lib.MoeTablesStruct._fields_] == fields


def test_tables_bytes_and_invalid_sizes():
    L = _lib.lib()
    assert L.moe_tables_bytes(512, 8, 256, 32) > 0
    assert L.moe_tables_bytes(0, 8, 256, 32) == 0
    assert L.moe_tables_bytes(512, 8, 256, 48) == 0       # block_m not a supported size
    assert L.moe_tables_bytes(512, 8, 2048, 32) == 0      # too many experts
    assert L.moe_tables_bytes(512, 65, 256, 32) == 0


def test_bind_layout_is_host_only_and_aligned():
    L = _lib.lib()
    s = _lib.MoeTablesStruct()
    n = L.moe_tables_bytes(100, 4, 16, 64)
    base = 1 << 20                         # a fake, never dereferenced address
    assert L.moe_tables_bind(ctypes.byref(s), ctypes.c_void_p(base), n, 100, 4, 16, 64) == 0
    assert s.num_blocks == -(-400 // 64) + 16
    ptrs = [getattr(s, f) for f, _ in _lib.MoeTablesStruct._fields_[6:]]
    assert all(p % 256 == 0 and base <= p < base + n for p in ptrs)
    assert len(set(ptrs)) == len(ptrs)
    assert L.moe_tables_bind(ctypes.byref(s), ctypes.c_void_p(base), n - 1, 100, 4, 16, 64) == 5
    assert L.moe_tables_bind(ctypes.byref(s), ctypes.c_void_p(base + 8), n, 100, 4, 16, 64) == 5
    assert L.moe_tables_bind(ctypes.byref(s), ctypes.c_void_p(base), n, 100, 4, 16, 24) == 4
    assert L.moe_tables_bind(None, ctypes.c_void_p(base), n, 100, 4, 16, 64) == 1


def test_calls_reject_bad_arguments_before_launching():
    L = _lib.lib()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    assert L.moe_dispatch(None, None, None, None) == 1
    assert L.moe_reduce_fused(None, 8, fake, None, 4, 2, 256, 1, 1, fake, None) == 1
    assert L.moe_reduce_fused(fake, 8, fake, None, 4, 2, 320, 1, 1, fake, None) == 2
    assert L.moe_reduce_fused(fake, 8, fake, None, 4, 0, 256, 1, 1, fake, None) == 2
    assert L.moe_reduce_fused(fake, 8, fake, None, 4, 2, 256, 7, 1, fake, None) == 3
    L.moe_reduce_fused(fake, 8, fake, None, 4, 2, 320, 1, 1, fake, None)
    assert "H must be" in L.moe_last_error().decode()
    s = _lib.MoeTablesStruct()   # unbound tables
    assert L.moe_routed_forward(fake, fake, fake, fake, ctypes.byref(s), 256, 128, 1, fake,
                                1 << 30, fake, None) == 1
    n = L.moe_tables_bytes(8, 2, 4, 32)
    assert L.moe_tables_bind(ctypes.byref(s), fake, n, 8, 2, 4, 32) == 0
    assert L.moe_routed_forward(fake, fake, fake, fake, ctypes.byref(s), 250, 128, 1, fake,
                                1 << 30, fake, None) == 2
    assert L.moe_routed_forward(fake, fake, fake, fake, ctypes.byref(s), 256, 100, 1, fake,
                                1 << 30, fake, None) == 2
    assert L.moe_routed_forward(fake, fake, fake, fake, ctypes.byref(s), 256, 128, 7, fake,
                                1 << 30, fake, None) == 3
    need = L.moe_forward_workspace_bytes(8, 2, 256, 128, 1)
    assert need > 0
    assert L.moe_routed_forward(fake, fake, fake, fake, ctypes.byref(s), 256, 128, 1, fake,
                                need - 1, fake, None) == 5
    assert L.moe_expert_gate_up(fake, fake, None, ctypes.byref(s), 256, 128, 1, fake, None) == 1
    assert L.moe_expert_down(fake, fake, ctypes.byref(s), 256, 128, 0, None, None) == 1
    assert L.moe_expert_down_weighted(fake, fake, ctypes.byref(s), 256, 128, 0, None, None) == 1
    assert L.moe_expert_down_weighted(fake, fake, ctypes.byref(s), 256, 100, 0, fake, None) == 2
    assert L.moe_routed_forward_weighted(fake, fake, fake, fake, ctypes.byref(s), 256, 128, 1,
                                         fake, need - 1, fake, None) == 5
    assert L.moe_routed_forward_weighted(fake, fake, fake, fake, ctypes.byref(s), 256, 128, 7,
                                         fake, 1 << 30, fake, None) == 3


def test_gate_rejects_bad_arguments_before_launching():
    L = _lib.lib()
    fake = ctypes.c_void_p(1 << 20)
    # moe_gate(x, w_router, bias, T, H, E, K, renorm, dtype, logits, ids, weights, stream)
    assert L.moe_gate(None, fake, None, 4, 64, 8, 2, 1, 1, fake, fake, fake, None) == 1
    assert L.moe_gate(fake, fake, None, 4, 64, 8, 2, 1, 1, None, fake, fake, None) == 1
    assert L.moe_gate(fake, fake, None, 4, 96, 8, 2, 1, 1, fake, fake, fake, None) == 2
    assert L.moe_gate(fake, fake, None, 4, 64, 2000, 2, 1, 1, fake, fake, fake, None) == 2
    assert L.moe_gate(fake, fake, None, 4, 64, 8, 9, 1, 1, fake, fake, fake, None) == 2
    assert L.moe_gate(fake, fake, None, 4, 64, 256, 65, 1, 1, fake, fake, fake, None) == 2
    assert L.moe_gate(fake, fake, None, -1, 64, 8, 2, 1, 1, fake, fake, fake, None) == 2
    assert L.moe_gate(fake, fake, None, 4, 64, 8, 2, 1, 3, fake, fake, fake, None) == 3
    assert "dtype" in L.moe_last_error().decode()
    assert L.moe_gate(fake, fake, None, 0, 64, 8, 2, 1, 1, fake, fake, fake, None) == 0


def test_workspace_layout():
    L = _lib.lib()
    T, K, H, D = 512, 8, 7168, 2048
    off = L.moe_forward_workspace_expert_out_offset(T, K, H, D, 1)
    assert off == T * K * D * 2
    assert L.moe_forward_workspace_bytes(T, K, H, D, 1) == off + T * K * H * 2


def test_default_block_m():
    assert mr.default_block_m(512, 8, 256) == 32      # ~16 rows per expert
    assert mr.default_block_m(512, 8, 128) == 64
    assert mr.default_block_m(4096, 8, 256) == 256
    assert mr.default_block_m(2048, 8, 256) == 128
    assert mr.default_block_m(1, 1, 256) == 16
    assert mr.default_block_m(4096, 8, 256, "w4a8") == 128
    assert mr.default_block_m(4096, 8, 256, "mx") == 64
    assert mr.default_block_m(4096, 8, 256, "w8a8") == 256
    assert mr.default_block_m(512, 8, 256, "mx") == 32


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_w4a8_calls_reject_bad_arguments_before_launching():
    L = _lib.lib()
    fake = ctypes.c_void_p(1 << 20)
    # moe_w4a8_gemm(A, B, M, N, K, Ct, stream)
    assert L.moe_w4a8_gemm(None, fake, 1, 256, 256, fake, None) == 1
    assert L.moe_w4a8_gemm(fake, fake, 0, 256, 256, fake, None) == 2
    assert L.moe_w4a8_gemm(fake, fake, 1, 200, 256, fake, None) == 2
    assert L.moe_w4a8_gemm(fake, fake, 1, 256, 300, fake, None) == 2
    assert L.moe_w4a8_gemm(fake, fake, 1, 256, 131072 + 256, fake, None) == 2
    assert "K must be" in L.moe_last_error().decode()
    # quantizers: odd row length for int4, bad dtype
    assert L.moe_quantize_int4_rows(fake, 4, 63, 1, fake, fake, None) == 2
    assert L.moe_quantize_int8_rows(fake, 4, 64, 3, fake, fake, None) == 3
    assert L.moe_quantize_int8_rows(fake, 0, 64, 1, fake, fake, None) == 0
    s = _lib.MoeTablesStruct()
    n = L.moe_tables_bytes(8, 2, 4, 32)
    assert L.moe_tables_bind(ctypes.byref(s), fake, n, 8, 2, 4, 32) == 0
    # moe_expert_gate_up_w4a8(xq, sx, wg, wu, sg, su, tables, H, D, dtype, h, stream)
    assert L.moe_expert_gate_up_w4a8(fake, fake, fake, fake, fake, fake, ctypes.byref(s), 256,
                                     128, 1, fake, None) == 2          # D % 256
    assert L.moe_expert_gate_up_w4a8(fake, fake, fake, fake, fake, fake, ctypes.byref(s), 256,
                                     256, 2, fake, None) == 3          # fp32 output
    assert L.moe_expert_down_w4a8(fake, None, fake, fake, ctypes.byref(s), 256, 256, 1, fake,
                                  None) == 1
    need = L.moe_forward_w4a8_workspace_bytes(8, 2, 256, 256, 1)
    assert need >= L.moe_forward_workspace_bytes(8, 2, 256, 256, 1) + 8 * 256 + 16 * 256
    assert L.moe_routed_forward_w4a8(fake, fake, fake, fake, fake, fake, fake, ctypes.byref(s),
                                     256, 256, 1, fake, need - 1, fake, None) == 5
