"""GPU parity of txl_rel_attn_fwd_mem_update (attention and ring append in one
launch) against the two separate calls (bit for bit) and the fp64 oracle.

The ring is the one the attention masks by (mem_valid is the ring's valid
array), so the test also checks that the valid counts advance only after the
attention has read them. Cases cover ragged segments and valid counts, L > M,
a ring dtype and width different from the attention's, appends much larger
than the grid's threads (the rounds after the key tiles), a single workgroup,
the bench layer, the fallback paths and the argument checks.
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import memory as om
from tests.gpu_helpers import assert_close, attn_case, f64, oracle_attn, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ring(x, B, M, d, dtype, head, g):
    """Ring whose logical slot j' holds mem_rows[b][j'] at physical slot (head + j') mod M."""
    logical = torch.randn((B, M, d), generator=g).to(dtype)
    data = torch.roll(logical, shifts=head, dims=1).contiguous() if M else logical
    mem = txl.TxlMem(data.to(DEV), x["valid"].to(DEV).clone(), head)
    rows = [f64(logical[b, M - int(x["valid"][b]):]) for b in range(B)]
    return mem, rows


def _clone(mem):
    return txl.TxlMem(mem.data.clone(), mem.valid.clone(), mem.head)


def _logical(mem):
    out = torch.empty_like(mem.data)
    txl.txl_mem_read_logical(mem, out)
    torch.cuda.synchronize()
    return out.cpu()


def _run_case(cfg, B, L, M, H, valid_mode, ring_dtype=torch.bfloat16, ring_d=None,
              head=0, steps=2, seed=5, use_valid=True, oracle=True):
    x = attn_case(cfg, B=B, L=L, M=M, H=H, seed=seed, valid_mode=valid_mode)
    d = ring_d if ring_d is not None else H * cfg.d_h
    say(f"fused B{B} H{H} L{L} M{M} ring {ring_dtype} d{d} head {head} valid={valid_mode}")
    g = torch.Generator().manual_seed(seed + 11)
    fused, rows = _ring(x, B, M, d, ring_dtype, head % M if M else 0, g)
    sep = _clone(fused)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    ws = txl.txl_rel_attn_mem_update_workspace(B)
    for step in range(steps):
        h = torch.randn((B, L, d), generator=g).to(ring_dtype)
        hd = h.to(DEV)
        valid_before = fused.valid.cpu().clone()
        out_f = torch.full((B, H, L, cfg.d_h), float("nan"), dtype=q.dtype, device=DEV)
        out_s = out_f.clone()
        lse_f = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=DEV)
        lse_s = lse_f.clone()
        txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out_f, fused, hd, ws,
                                        mem_valid=fused.valid if use_valid else None, lse=lse_f)
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out_s, mem_valid=sep.valid if use_valid else None,
                             lse=lse_s)
        txl.txl_mem_update([sep], [hd])
        torch.cuda.synchronize()
        assert torch.equal(out_f.cpu(), out_s.cpu()), f"step {step}: out differs"
        assert torch.equal(lse_f.cpu(), lse_s.cpu()), f"step {step}: lse differs"
        assert torch.equal(fused.data.cpu(), sep.data.cpu()), f"step {step}: ring slots differ"
        assert torch.equal(fused.valid.cpu(), sep.valid.cpu()), f"step {step}: valid differs"
        assert fused.head == sep.head
        assert (ws.cpu() == 0).all(), "workspace counters not returned to zero"
        if oracle:
            # the attention saw the valid counts from before the call
            xs = dict(x)
            xs["valid"] = valid_before if use_valid else torch.full((B,), M, dtype=torch.int32)
            ref = oracle_attn(xs)
            assert_close(cfg.dtype, f64(out_f), ref["out"], f"fused step {step} out")
            if M:
                rows = om.update_rows(rows, f64(h), M)
                logi = _logical(fused)
                valid = fused.valid.cpu().numpy()
                for b in range(B):
                    assert valid[b] == rows[b].shape[0], (b, valid[b], rows[b].shape)
                    got = logi[b, M - valid[b]:].double().numpy()
                    assert np.array_equal(got, rows[b]), f"step {step} ring row {b}"
        # the next step attends with the advanced counts, as a stream would
        x = dict(x)
        x["valid"] = fused.valid.cpu().clone()


CFG = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]


@pytest.mark.parametrize("valid_mode", ["full", "mixed", "empty"])
def test_fused_layer_with_memory(valid_mode):
    _run_case(CFG, B=4, L=128, M=128, H=8, valid_mode=valid_mode, head=37)


def test_fused_ragged_segment():
    _run_case(CFG, B=3, L=50, M=70, H=2, valid_mode="mixed", head=69, steps=3)


def test_fused_segment_longer_than_memory():
    # L > M: only the last M rows of the segment are appended
    _run_case(CFG, B=2, L=200, M=64, H=2, valid_mode="mixed", head=10)


@pytest.mark.parametrize("L,M", [(300, 100), (600, 40)])
def test_fused_odd_query_tile_counts(L, M):
    # 3 and 5 query tiles of 128: the copy goes to the lighter 1 and 2 of them
    _run_case(CFG, B=2, L=L, M=M, H=2, valid_mode="mixed", head=M - 1, steps=2)


def test_fused_fp32_wide_ring_many_rounds():
    # ring width and dtype independent of the attention: 16 KiB rows, two
    # workgroups, so nearly all rounds run after the key tiles
    _run_case(CFG, B=2, L=100, M=300, H=1, valid_mode="mixed", ring_dtype=torch.float32,
              ring_d=4096, head=299)


def test_fused_single_workgroup():
    _run_case(CFG, B=1, L=24, M=40, H=1, valid_mode="full", head=3, steps=3)


def test_fused_without_mem_valid():
    _run_case(CFG, B=2, L=64, M=96, H=4, valid_mode="mixed", head=1, use_valid=False)


def test_fused_bench_layer():
    """The benchmark's step at full size (B8 H16 L512 M512): bit-identical
    to the two calls, every (batch row, head) slice against the oracle, the
    ring against Tail_M, over two consecutive steps."""
    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    _run_case(cfg, B=8, L=512, M=512, H=16, valid_mode="full", head=0, steps=2, seed=1)


def test_fused_fp32_attention_falls_back():
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32"]
    _run_case(cfg, B=3, L=4, M=8, H=1, valid_mode="mixed", ring_dtype=torch.float32, head=5)


def test_fused_zero_memory_is_attention_only():
    x = attn_case(CFG, B=2, L=64, M=0, H=2, seed=3)
    mem = txl.TxlMem.empty(2, 0, 128)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    out_f = torch.empty((2, 2, 64, 64), dtype=torch.bfloat16, device=DEV)
    out_s = torch.empty_like(out_f)
    ws = txl.txl_rel_attn_mem_update_workspace(2)
    h = torch.randn((2, 64, 128), device=DEV).to(torch.bfloat16)
    txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out_f, mem, h, ws, mem_valid=mem.valid)
    txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out_s)
    torch.cuda.synchronize()
    assert torch.equal(out_f.cpu(), out_s.cpu())
    assert mem.head == 0 and (mem.valid.cpu() == 0).all()


def test_fused_empty_segment_is_noop():
    x = attn_case(CFG, B=2, L=8, M=16, H=2, seed=6)
    mem = txl.TxlMem(torch.ones((2, 16, 128), dtype=torch.bfloat16, device=DEV),
                     torch.full((2,), 5, dtype=torch.int32, device=DEV), 3)
    q = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    k = x["k"][:, :, :16].to(DEV)
    r = x["r"][:, :16].to(DEV)
    out = torch.empty_like(q)
    h = torch.empty((2, 0, 128), dtype=torch.bfloat16, device=DEV)
    ws = txl.txl_rel_attn_mem_update_workspace(2)
    txl.txl_rel_attn_fwd_mem_update(q, k, k, r, x["u"].to(DEV), x["vb"].to(DEV), out, mem, h, ws,
                                    mem_valid=mem.valid)
    torch.cuda.synchronize()
    assert mem.head == 3 and (mem.valid.cpu() == 5).all() and (mem.data.cpu() == 1).all()


def test_fused_rejects_bad_arguments():
    x = attn_case(CFG, B=2, L=32, M=16, H=2, seed=4)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    out = torch.empty((2, 2, 32, 64), dtype=torch.bfloat16, device=DEV)
    h = torch.zeros((2, 32, 128), dtype=torch.bfloat16, device=DEV)
    ws = txl.txl_rel_attn_mem_update_workspace(2)
    wrong_m = txl.TxlMem.empty(2, 17, 128)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out, wrong_m, h, ws)
    assert e.value.status_name == "TXL_ERR_INVALID_ARG"
    mem = txl.TxlMem.empty(2, 16, 128)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out, mem, h,
                                        torch.zeros(256, dtype=torch.uint8, device=DEV))
    assert e.value.status_name == "TXL_ERR_WORKSPACE"
    assert mem.head == 0 and (mem.valid.cpu() == 0).all()
