"""GPU tests of txl_segment_step_kv: memory kept as projected keys / values.

With fixed weights, keeping each layer's memory as K = mem W^K, V = mem W^V
gives the same keys and values as projecting the stored hidden states again
every segment ([P1] "Relation to KV Cache" contrasts the two). The library's
GEMM accumulates every output element in the same order whatever the row
count and tile shape, so the two paths must agree bit for bit: the ring path
(txl_segment_step, itself checked against the fp64 oracle layer by layer) is
the reference here, over streams with per-row resets and window compactions.
A one-layer stream is also checked directly against the oracle.
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import stack as ost
from tests.gpu_helpers import f64, say
from tests.test_gpu_stack import ATOL, RTOL, make_stack

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cfg_of(M, L, B=3, n_layer=2, seed=3, n_seg=8, reset_every=0):
    return txl_synth.StackConfig("kv", "bf16", n_layer=n_layer, d=256, H=4, d_h=64, d_ff=512,
                                 vocab=97, B=B, L=L, M=M, n_seg=n_seg, seed=seed, w_std=0.05,
                                 reset_every=reset_every)


def kv_caches(st, cfg, capacity):
    hd = cfg.H * cfg.d_h
    return [txl.TxlKVCache.empty(cfg.B, capacity, hd) for _ in range(cfg.n_layer)]


def both_streams(cfg, capacity, resets, tokens=None, w=None):
    """Run the ring path and the projected-memory path side by side; returns
    the number of segments compared and of compactions seen."""
    w = w if w is not None else txl_synth.stack_weights(cfg)
    tokens = tokens if tokens is not None else txl_synth.stack_tokens(cfg)
    st, keep = make_stack(cfg, w)
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    caches = kv_caches(st, cfg, capacity)
    h_ring = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    h_kv = torch.empty_like(h_ring)
    compactions = 0
    for s in range(tokens.shape[0]):
        tok = tokens[s].to(DEV).contiguous()
        if resets[s].any():
            r = resets[s].to(DEV).contiguous()
            txl.txl_mem_reset_rows(mems, r)
            txl.txl_kv_cache_reset_rows(caches, r)
        before = caches[0].start
        st.step(tok, mems, h_ring)
        st.step_kv(tok, caches, h_kv)
        torch.cuda.synchronize()
        if caches[0].start < before:
            compactions += 1
        assert all(c.start == caches[0].start for c in caches)
        for n in range(cfg.n_layer):
            assert torch.equal(caches[n].valid, mems[n].valid), (s, n)
        same = torch.equal(h_ring, h_kv)
        if not same:
            diff = (h_ring.float() - h_kv.float()).abs().max().item()
            say(f"segment {s}: max |ring - kv| {diff:.3e}")
        assert same, s
    st.close()
    del keep
    return tokens.shape[0], compactions


@pytest.mark.parametrize("M,L,extra", [(64, 32, 0), (96, 64, 2), (32, 64, 1), (0, 32, 0)])
def test_kv_stream_equals_ring_stream_bitwise(M, L, extra):
    """Streams of 8 segments with per-row resets; capacity 2M + L (+ extra
    segments) so that the window is compacted several times."""
    cfg = cfg_of(M, L)
    resets = torch.zeros((cfg.n_seg, cfg.B), dtype=torch.uint8)
    resets[3, 1] = 1
    resets[5, :] = 1
    resets[6, 2] = 1
    cap = 2 * M + L + extra * L
    n, comp = both_streams(cfg, cap, resets)
    say(f"M={M} L={L} capacity={cap}: {n} segments bit-identical, {comp} compactions")
    if M > 0:
        assert comp >= 2


def test_kv_one_layer_stream_against_oracle():
    """One layer, so the memory the oracle needs is the embedding of earlier
    tokens (exact): every segment's output checked against the fp64 layer."""
    cfg = cfg_of(64, 32, B=2, n_layer=1, seed=9, n_seg=6)
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    st, keep = make_stack(cfg, w)
    caches = kv_caches(st, cfg, 2 * cfg.M + cfg.L)
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    emb = f64(w["emb"])
    lw = {k: f64(t) for k, t in w["layers"][0].items()}
    r = ost.rel_pos_table(lw["wr"], cfg.M, cfg.L, cfg.H, cfg.d_h)
    history = [np.zeros((0, cfg.d)) for _ in range(cfg.B)]
    reset_at = {3: [1]}
    worst = 0.0
    for s in range(cfg.n_seg):
        if s in reset_at:
            rr = torch.zeros(cfg.B, dtype=torch.uint8)
            rr[reset_at[s]] = 1
            txl.txl_kv_cache_reset_rows(caches, rr.to(DEV))
            for b in reset_at[s]:
                history[b] = np.zeros((0, cfg.d))
        st.step_kv(tokens[s].to(DEV).contiguous(), caches, h)
        torch.cuda.synchronize()
        got = f64(h)
        for b in range(cfg.B):
            h0 = emb[tokens[s, b].numpy()]
            mem = history[b][-cfg.M:] if cfg.M else history[b][:0]
            ref = ost.layer_forward(h0, mem, lw, r, cfg.M, cfg.H, cfg.d_h)
            err = np.abs(got[b] - ref)
            worst = max(worst, float(err.max()))
            assert (err <= ATOL + RTOL * np.abs(ref)).all(), (s, b, float(err.max()))
            history[b] = np.concatenate([history[b], h0], axis=0)
    say(f"one-layer projected-memory stream: max abs err {worst:.3e}")
    st.close()
    del keep


def test_kv_eighteen_layers_full_size_equals_ring_bitwise():
    """18 layers, d=1024, B=8, L=128, M=640, 16 segments with every row
    resetting at segments 0, 4, 8, 12; capacity 2M + L (compaction every six
    segments)."""
    cfg = txl_synth.STACK_CONFIGS["18layer_d1024"]
    resets = txl_synth.reset_schedule(cfg)
    n, comp = both_streams(cfg, 2 * cfg.M + cfg.L, resets)
    say(f"18 layers: {n} segments bit-identical, {comp} compactions")
    assert comp >= 2


def test_kv_step_rejects_bad_arguments():
    cfg = cfg_of(64, 32)
    w = txl_synth.stack_weights(cfg)
    st, keep = make_stack(cfg, w)
    assert st.kv_min_capacity() == 2 * 64 + 32
    tok = torch.zeros((cfg.B, cfg.L), dtype=torch.int32, device=DEV)
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)

    def expect(caches, status):
        with pytest.raises(txl.TxlError) as e:
            st.step_kv(tok, caches, h)
        assert e.value.status_name == status

    expect(kv_caches(st, cfg, 2 * 64 + 31), "TXL_ERR_INVALID_ARG")       # too small
    caches = kv_caches(st, cfg, 200)
    for c in caches:
        c.start = 200 - 64 - 32 + 1                                        # window past the end
    expect(caches, "TXL_ERR_INVALID_ARG")
    caches = kv_caches(st, cfg, 200)
    caches[1].start = 32                                                   # starts differ
    expect(caches, "TXL_ERR_INVALID_ARG")
    caches = kv_caches(st, cfg, 200)
    caches[1] = txl.TxlKVCache.empty(cfg.B, 240, cfg.H * cfg.d_h)         # capacities differ
    expect(caches, "TXL_ERR_INVALID_ARG")
    caches = kv_caches(st, cfg, 200)
    caches[0] = txl.TxlKVCache.empty(cfg.B, 200, 2 * cfg.H * cfg.d_h)     # wrong width
    expect(caches, "TXL_ERR_INVALID_ARG")
    caches = kv_caches(st, cfg, 200)
    assert all(c.start == 0 for c in caches)
    st.close()
    del keep
    odd = cfg_of(64, 40)                                                   # L not a multiple of 32
    st2, keep2 = make_stack(odd, txl_synth.stack_weights(odd))
    tok2 = torch.zeros((odd.B, odd.L), dtype=torch.int32, device=DEV)
    h2 = torch.empty((odd.B, odd.L, odd.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(txl.TxlError) as e:
        st2.step_kv(tok2, kv_caches(st2, odd, 2 * 64 + 40), h2)
    assert e.value.status_name == "TXL_ERR_UNSUPPORTED"
    st2.close()
    del keep2
