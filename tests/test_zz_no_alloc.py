"""The attention + ring append entry point that allocates nothing
(txl_rel_attn_fwd_mem_update_noalloc) against the one that takes a
workspace (txl_rel_attn_fwd_mem_update), through the C ABI: out, lse, ring
slots, valid counts and head bit for bit, on two calls in a row, the second
with a smaller input (the static counters are shared by every call on the
GPU and must be left clean by the first).
"""
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from tests.gpu_helpers import attn_case, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]


def _call_pair(B, H, L, M, head, seed):
    say(f"no-alloc vs workspace: B{B} H{H} L{L} M{M} head {head}")
    x = attn_case(CFG, B=B, L=L, M=M, H=H, seed=seed, valid_mode="mixed")
    d = H * CFG.d_h
    g = torch.Generator().manual_seed(seed + 3)
    data = torch.randn((B, M, d), generator=g).to(torch.bfloat16).to(DEV)
    ring_a = txl.TxlMem(data.clone(), x["valid"].to(DEV).clone(), head)
    ring_b = txl.TxlMem(data.clone(), x["valid"].to(DEV).clone(), head)
    h = torch.randn((B, L, d), generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    out_a = torch.full((B, H, L, CFG.d_h), float("nan"), dtype=torch.bfloat16, device=DEV)
    out_b = out_a.clone()
    lse_a = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=DEV)
    lse_b = lse_a.clone()
    ws = txl.txl_rel_attn_mem_update_workspace(B)
    txl.txl_rel_attn_fwd_mem_update_noalloc(q, k, v, r, u, vb, out_a, ring_a, h,
                                            mem_valid=ring_a.valid, lse=lse_a)
    txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out_b, ring_b, h, ws,
                                    mem_valid=ring_b.valid, lse=lse_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.cpu(), out_b.cpu()), "out differs"
    assert torch.equal(lse_a.cpu(), lse_b.cpu()), "lse differs"
    assert torch.equal(ring_a.data.cpu(), ring_b.data.cpu()), "ring slots differ"
    assert torch.equal(ring_a.valid.cpu(), ring_b.valid.cpu()), "valid counts differ"
    assert ring_a.head == ring_b.head == (head + min(L, M)) % M
    assert torch.isfinite(out_a.float()).all()


def test_noalloc_equals_workspace_call_twice_second_smaller():
    _call_pair(B=8, H=8, L=256, M=192, head=17, seed=41)
    _call_pair(B=3, H=2, L=50, M=70, head=69, seed=42)


def test_noalloc_bench_shape_then_small():
    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    del cfg
    _call_pair(B=8, H=16, L=512, M=512, head=0, seed=43)
    _call_pair(B=1, H=1, L=24, M=40, head=3, seed=44)
