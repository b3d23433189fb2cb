"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


def _declared():
    names = []
    for h in HEADERS:
        text = open(h).read()
        names += re.findall(r"TXL_API\s+[\w\s\*]+?\b(txl_\w+)\s*\(", text)
    return names


@pytest.fixture(scope="module")
def lib():
    from transformer_xl_relative_txl_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    from transformer_xl_relative_txl_amd import _binding
    return _binding.lib()


def test_header_declares_entry_points():
    names = _declared()
    for n in ("txl_rel_attn_fwd", "txl_mem_update", "txl_rel_pos_table",
              "txl_mem_reset_rows", "txl_mem_read_logical"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert lib.txl_version() == 1
    assert lib.txl_status_str(0) == b"ok"
    assert lib.txl_status_str(2) == b"unsupported"


def test_null_and_bad_sizes_rejected_without_gpu(lib):
    from transformer_xl_relative_txl_amd import _binding as bd
    assert lib.txl_rel_attn_fwd(None, None) == 1
    assert b"null args" in lib.txl_last_error()
    a = bd.RelAttnArgs()
    a.dtype, a.B, a.H, a.L, a.M, a.d_h = 1, 1, 1, 4, 8, 32
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 2      # d_h unsupported
    a.d_h, a.L = 64, -1
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 1      # negative L
    a.L = 4
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 1      # null tensors
    a.dtype = 7
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 1      # bad dtype
    assert lib.txl_rel_pos_table(1, 8, 4, 63, 1, 64, None, None, None) == 1  # odd d
    assert lib.txl_mem_update(None, -1, None, 4, None) == 1
    assert lib.txl_mem_reset_rows(None, -1, None, None) == 1
    assert lib.txl_mem_read_logical(None, None, None) == 1


def test_stack_and_kv_cache_host_checks_without_gpu(lib):
    from transformer_xl_relative_txl_amd import _binding as bd
    cfg = bd.StackConfig(2, 256, 4, 64, 256, 50, 2, 32, 64, 1e-5, bd.TXL_BF16)
    assert lib.txl_kv_cache_min_capacity(ctypes.byref(cfg)) == 2 * 64 + 32
    bad = bd.StackConfig(2, 256, 4, 32, 256, 50, 2, 32, 64, 1e-5, bd.TXL_BF16)  # d_h 32
    assert lib.txl_kv_cache_min_capacity(ctypes.byref(bad)) == 0
    assert lib.txl_segment_step_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.txl_segment_step_kv(None, None, None, None, None, 0, None) == 1
    assert lib.txl_segment_step(None, None, None, None, None, 0, None) == 1
    assert lib.txl_kv_cache_reset_rows(None, -1, None, None) == 1
    assert lib.txl_kv_cache_reset_rows(None, 0, None, None) == 0       # nothing to do
    arr = (bd.TxlKVCacheStruct * 2)()
    arr[0].B, arr[1].B = 2, 3
    assert lib.txl_kv_cache_reset_rows(arr, 2, None, None) == 1        # B differs
    assert b"differ in B" in lib.txl_last_error()
    arr[1].B = 2
    assert lib.txl_kv_cache_reset_rows(arr, 2, None, None) == 1        # null valid
