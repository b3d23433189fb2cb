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
    assert lib.txl_mem_update(None, -1, None, 0, 4, None) == 1
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


def test_stream_sampler_equals_oracle_bitwise(lib):
    """The library's host sampler against the oracle's reading of the stream
    contract, on random documents: tokens, targets, resets and lengths equal."""
    import numpy as np
    from oracle import evaluation as ev
    from transformer_xl_relative_txl_amd import _binding as bd
    rng = np.random.default_rng(5)
    for B, L, n_docs, max_len in [(4, 8, 5, 40), (3, 64, 3, 200), (2, 1, 2, 3)]:
        docs = [[rng.integers(1, 1000, size=int(rng.integers(1, max_len + 1))).tolist()
                 for _ in range(n_docs)] for _ in range(B)]
        n_seg = 50
        t, g, r, n = ev.row_streams(docs, L, n_seg, pad_id=7)
        s = bd.StreamSampler(docs, L, pad_id=7)
        for k in range(n_seg):
            tok, tgt, rst, ln = s.next()
            assert (tok == t[k]).all() and (tgt == g[k]).all(), (B, L, k)
            assert (rst == r[k]).all() and (ln == n[k]).all(), (B, L, k)
        s.close()


def test_stream_sampler_and_loss_reject_bad_arguments(lib):
    import numpy as np
    from transformer_xl_relative_txl_amd import _binding as bd
    tok = np.arange(10, dtype=np.int32)
    off = np.array([0, 4, 4, 10], dtype=np.int64)        # document 1 is empty
    ro = np.array([0, 1], dtype=np.int32)
    rd = np.array([0], dtype=np.int32)
    h = ctypes.c_void_p()
    assert lib.txl_sampler_create(1, 4, tok.ctypes.data, off.ctypes.data, 3, ro.ctypes.data,
                                  rd.ctypes.data, 0, ctypes.byref(h)) == 1
    assert b"empty" in lib.txl_last_error()
    off = np.array([0, 4, 10], dtype=np.int64)
    rd = np.array([5], dtype=np.int32)                     # no such document
    assert lib.txl_sampler_create(1, 4, tok.ctypes.data, off.ctypes.data, 2, ro.ctypes.data,
                                  rd.ctypes.data, 0, ctypes.byref(h)) == 1
    ro = np.array([0, 0], dtype=np.int32)                  # row without documents
    assert lib.txl_sampler_create(1, 4, tok.ctypes.data, off.ctypes.data, 2, ro.ctypes.data,
                                  rd.ctypes.data, 0, ctypes.byref(h)) == 1
    assert lib.txl_sampler_next(None, None, None, None, None) == 1
    # loss: checks before any launch
    assert lib.txl_lm_loss(None, None, None, 0, 64, 100, None, None, 0, None) == 0   # nothing to do
    assert lib.txl_lm_loss(None, None, None, 64, 64, 100, None, None, 0, None) == 1  # null
    fake = 1 << 20
    assert lib.txl_lm_loss(fake, fake, fake, 65, 64, 100, fake, fake, 1 << 30, None) == 2
    assert lib.txl_lm_loss(fake, fake, fake, 64, 48, 100, fake, fake, 1 << 30, None) == 2
    assert lib.txl_lm_loss(fake, fake, fake, 64, 64, 100, fake, fake, 16, None) == 3  # workspace
    assert lib.txl_lm_loss_workspace_bytes(64, 100) >= 2 * 64 * 4 + 64 * 4


def test_attention_backward_checks_without_gpu(lib):
    """The gradient entry point validates before launching: fake but aligned
    device addresses are never dereferenced on these error paths."""
    from transformer_xl_relative_txl_amd import _binding as bd
    a = bd.RelAttnArgs()
    a.dtype, a.B, a.H, a.L, a.M, a.d_h = 1, 2, 3, 64, 32, 64
    fake = 1 << 20
    a.q = a.k = a.v = a.r = a.u = a.vb = a.out = fake
    a.q_sb, a.q_sh, a.q_sl = 3 * 64 * 64, 64 * 64, 64
    a.kv_sb, a.kv_sh, a.kv_sl = 3 * 96 * 64, 96 * 64, 64
    a.r_sh, a.r_sl = 96 * 64, 64
    a.o_sb, a.o_sh, a.o_sl = a.q_sb, a.q_sh, a.q_sl
    g = bd.RelAttnGrads()
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), None, None, 0, None) == 1       # null grads
    a.lse = None
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), None, 0, None) == 1  # no lse
    a.lse = fake
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), None, 0, None) == 1  # null outputs
    g.dout = g.dq = g.dk = g.dv = g.dr = g.du = g.dvb = fake
    g.do_sb, g.do_sh, g.do_sl = a.q_sb, a.q_sh, a.q_sl
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), None, 0, None) == 3  # workspace
    need = lib.txl_rel_attn_bwd_workspace_bytes(2, 3, 64, 32)
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), fake, need - 1, None) == 3
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), fake + 16, need, None) == 2
    g.do_sl = 65                                                                 # odd stride
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), fake, need, None) == 2
    g.do_sl = 64
    a.dtype = 0                                                                  # fp32 inputs
    assert lib.txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), fake, need, None) == 2
    assert b"bf16" in lib.txl_last_error()
    # p and g rows of (M + L) rounded up to 8 elements dominate the workspace
    ldp = (32 + 64 + 7) // 8 * 8
    assert need >= 2 * 2 * 3 * 64 * ldp * 2
    assert lib.txl_rel_attn_bwd_workspace_bytes(-1, 3, 64, 32) == 0
    # the unrounded output: bf16 only, 16-byte aligned
    a.out_f32 = fake + 4
    a.dtype = 1
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 2
    assert b"out_f32" in lib.txl_last_error()
    a.out_f32, a.dtype = fake, 0
    assert lib.txl_rel_attn_fwd(ctypes.byref(a), None) == 2
    assert b"out_f32" in lib.txl_last_error()


def test_attention_with_ring_append_checks_without_gpu(lib):
    """The fused attention + ring append validates before launching: fake
    but aligned device addresses are never dereferenced on these error paths,
    and the ring's host head is left alone when a call is rejected."""
    from transformer_xl_relative_txl_amd import _binding as bd
    a = bd.RelAttnArgs()
    a.dtype, a.B, a.H, a.L, a.M, a.d_h = 1, 2, 3, 64, 32, 64
    fake = 1 << 20
    a.q = a.k = a.v = a.r = a.u = a.vb = a.out = fake
    a.q_sb, a.q_sh, a.q_sl = 3 * 64 * 64, 64 * 64, 64
    a.kv_sb, a.kv_sh, a.kv_sl = 3 * 96 * 64, 96 * 64, 64
    a.r_sh, a.r_sl = 96 * 64, 64
    a.o_sb, a.o_sh, a.o_sl = a.q_sb, a.q_sh, a.q_sl
    m = bd.TxlMemStruct()
    m.data, m.valid, m.head, m.B, m.M, m.d, m.dtype = fake, fake, 7, 2, 32, 192, 1
    need = lib.txl_rel_attn_mem_update_workspace_bytes(2)
    assert need == 2 * 256 and lib.txl_rel_attn_mem_update_workspace_bytes(0) == 0
    call = lambda ring, h, ws, n: lib.txl_rel_attn_fwd_mem_update(
        ctypes.byref(a), ring, h, ws, n, None)
    assert call(None, fake, fake, need) == 1                          # no ring
    assert call(ctypes.byref(m), None, fake, need) == 1               # no h
    assert call(ctypes.byref(m), fake, None, need) == 3               # no workspace
    assert call(ctypes.byref(m), fake, fake, need - 1) == 3           # workspace too small
    assert call(ctypes.byref(m), fake, fake + 16, need) == 2          # workspace not 256-aligned
    assert call(ctypes.byref(m), fake + 8, fake, need) == 2           # h not 16-byte aligned
    m.d = 100                                                         # row of 200 bytes
    assert call(ctypes.byref(m), fake, fake, need) == 2
    m.d, m.M = 192, 33                                                # capacity != attention's M
    assert call(ctypes.byref(m), fake, fake, need) == 1
    m.M, m.B = 32, 3                                                  # rows != attention's B
    assert call(ctypes.byref(m), fake, fake, need) == 1
    assert m.head == 7                                                # untouched by rejections
    m.B, m.head = 2, 32                                               # head outside [0, M)
    assert call(ctypes.byref(m), fake, fake, need) == 1


def test_mem_update_row_stride_checks_without_gpu(lib):
    """h_row_stride is checked on the host before anything is launched (the
    device pointers below are never dereferenced)."""
    from transformer_xl_relative_txl_amd import _binding as bd
    ring = bd.TxlMemStruct()
    ring.data, ring.valid, ring.head = 4096, 4096, 0
    ring.B, ring.M, ring.d, ring.dtype = 2, 4, 16, bd.TXL_F32
    h = (ctypes.c_void_p * 1)(8192)
    assert lib.txl_mem_update(ctypes.byref(ring), 1, h, 8, 3, None) == 1      # stride < d
    assert b"h_row_stride" in lib.txl_last_error()
    assert lib.txl_mem_update(ctypes.byref(ring), 1, h, 18, 3, None) == 2     # 72-byte rows
    assert lib.txl_mem_update(ctypes.byref(ring), 1, h, -1, 3, None) == 1
    assert ring.head == 0


def test_noalloc_attention_append_host_checks_without_gpu(lib):
    """The no-alloc entry point rejects batch counts beyond its static
    counters, and the usual argument errors, before anything is launched
    (the pointers below are never dereferenced)."""
    from transformer_xl_relative_txl_amd import _binding as bd
    a = bd.RelAttnArgs()
    a.dtype, a.B, a.H, a.L, a.M, a.d_h = bd.TXL_BF16, 4097, 1, 8, 8, 64
    for n in ("q", "k", "v", "r", "u", "vb", "out"):
        setattr(a, n, 4096)
    a.q_sl = a.kv_sl = a.r_sl = a.o_sl = 64
    ring = bd.TxlMemStruct()
    ring.data, ring.valid, ring.head = 4096, 4096, 0
    ring.B, ring.M, ring.d, ring.dtype = 4097, 8, 64, bd.TXL_BF16
    st = lib.txl_rel_attn_fwd_mem_update_noalloc(ctypes.byref(a), ctypes.byref(ring), 8192, None)
    assert st == 2 and b"4096" in lib.txl_last_error()
    ring.M = 9                                          # ring differs from the attention
    assert lib.txl_rel_attn_fwd_mem_update_noalloc(ctypes.byref(a), ctypes.byref(ring),
                                                   8192, None) == 1
    assert lib.txl_rel_attn_fwd_mem_update_noalloc(None, None, None, None) == 1
    assert ring.head == 0


def test_training_entry_points_host_checks_without_gpu(lib):
    from transformer_xl_relative_txl_amd import _binding as bd
    cfg = bd.StackConfig(2, 256, 4, 64, 512, 50, 2, 32, 64, 1e-5, bd.TXL_BF16)
    tape = lib.txl_segment_tape_bytes(ctypes.byref(cfg))
    ws = lib.txl_segment_backward_workspace_bytes(ctypes.byref(cfg))
    rows, krows, hd = 2 * 32, 2 * (64 + 32), 256
    # the tape holds at least H, Q, K, V, A, both LayerNorm inputs and the
    # feed-forward's two [rows, d_ff] products of every layer
    per_layer = rows * 256 * 2 + rows * hd * 2 * 2 + krows * hd * 2 * 2 + rows * 256 * 4 * 2 \
        + rows * 512 * 2 * 2
    assert tape >= 2 * per_layer and tape % 256 == 0
    assert ws > 0 and ws % 256 == 0
    bad = bd.StackConfig(2, 256, 4, 32, 256, 50, 2, 32, 64, 1e-5, bd.TXL_BF16)  # d_h 32
    assert lib.txl_segment_tape_bytes(ctypes.byref(bad)) == 0
    assert lib.txl_segment_backward_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.txl_segment_step_train(None, None, None, None, None, 0, None, 0, None) == 1
    assert lib.txl_segment_backward(None, None, 0, None, None, None, 0, None) == 1
    assert b"null" in lib.txl_last_error()
