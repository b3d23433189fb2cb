"""GPU parity of txl_lm_loss (segment cross entropy, logits never stored)
against the fp64 oracle on the same bf16 inputs, and an evaluation stream:
sampler -> resets -> stack step -> loss.

Tolerance: the GPU and the oracle see the same bf16 h and w_out; the GPU
accumulates each logit in fp32 over d terms (relative error about d * 2^-24
of the sum of |terms|) and evaluates exp / log with the hardware's fp32
instructions (a few ulp), so the loss agrees to
    |gpu - ref| <= 1e-4 + 1e-5 |ref|
at the sizes here (d <= 512, logits of order 1-10).
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import evaluation as ev
from tests.gpu_helpers import f64, say
from tests.test_gpu_stack import make_stack

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL, RTOL = 1e-4, 1e-5


def draw(n_tok, d, vocab, seed, w_std=1.0):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn((n_tok, d), generator=g).to(torch.bfloat16)
    w = (torch.randn((vocab, d), generator=g) * w_std / d ** 0.5).to(torch.bfloat16)
    tg = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    return h, w, tg


def run(h, w, tg):
    nll = torch.empty(h.shape[0], dtype=torch.float32, device=DEV)
    txl.txl_lm_loss(h.to(DEV), w.to(DEV), tg.to(DEV), nll)
    torch.cuda.synchronize()
    return nll.cpu().double().numpy()


def check(got, ref, what):
    err = np.abs(got - ref)
    say(f"{what}: max abs err {err.max():.2e} (max loss {np.abs(ref).max():.2f})")
    assert (err <= ATOL + RTOL * np.abs(ref)).all(), what


@pytest.mark.parametrize("n_tok,d,vocab,seed", [(128, 64, 97, 0), (192, 256, 1000, 1),
                                                (64, 32, 1, 2), (256, 128, 4097, 3)])
def test_loss_small_all_tokens(n_tok, d, vocab, seed):
    """Ragged vocabularies (one entry, 97, 4097: partial 128-row tiles) and
    token counts that are not multiples of 128 (64-wide token tiles)."""
    h, w, tg = draw(n_tok, d, vocab, seed, w_std=3.0)
    tg[::5] = -1                      # no target
    tg[3] = vocab                     # outside the vocabulary: ignored too
    got = run(h, w, tg)
    ref = ev.segment_nll(f64(h), f64(w), np.where(tg.numpy() >= vocab, -1, tg.numpy()))
    check(got, ref, f"n_tok {n_tok} d {d} vocab {vocab}")
    assert (got[::5] == 0).all() and got[3] == 0


def test_loss_sixteen_layer_shape_sampled():
    """The 16-layer workload's segment: 16 x 384 tokens, d = 512, vocabulary
    32768 (12288 tiles); 96 tokens checked against the oracle, every token
    checked to be finite and non-negative."""
    n_tok, d, vocab = 16 * 384, 512, 32768
    h, w, tg = draw(n_tok, d, vocab, 4, w_std=2.0)
    got = run(h, w, tg)
    assert np.isfinite(got).all() and (got >= -1e-4).all()
    idx = np.random.default_rng(0).choice(n_tok, 96, replace=False)
    ref = ev.segment_nll(f64(h[idx]), f64(w), tg.numpy()[idx])
    check(got[idx], ref, "16x384 tokens, vocab 32768 (sampled)")


def test_loss_zero_weights_is_log_vocab():
    n_tok, d, vocab = 64, 64, 300
    h, _, tg = draw(n_tok, d, vocab, 5)
    w = torch.zeros((vocab, d), dtype=torch.bfloat16)
    got = run(h, w, tg)
    assert np.allclose(got, np.log(vocab), rtol=0, atol=1e-5)


def test_loss_rejects_bad_arguments():
    h = torch.zeros((96, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((50, 64), dtype=torch.bfloat16, device=DEV)
    tg = torch.zeros(96, dtype=torch.int32, device=DEV)
    nll = torch.empty(96, dtype=torch.float32, device=DEV)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_lm_loss(h, w, tg, nll)             # 96 tokens: not a multiple of 64
    assert e.value.status_name == "TXL_ERR_UNSUPPORTED"
    h2 = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_lm_loss(h2, w, tg[:64], nll[:64], workspace=ws)
    assert e.value.status_name == "TXL_ERR_WORKSPACE"


def test_evaluation_stream_sampler_stack_loss():
    """Documents of random lengths stream through a 2-layer stack: the
    sampler's reset flags clear rows' memories, the step runs, and the loss of
    every segment (tied output embedding) matches the oracle's cross entropy
    of the GPU's own h_out; padded positions and document ends add nothing."""
    cfg = txl_synth.StackConfig("eval", "bf16", n_layer=2, d=256, H=4, d_h=64, d_ff=512,
                                vocab=211, B=4, L=32, M=64, n_seg=10, seed=8, w_std=0.05,
                                reset_every=0)
    w = txl_synth.stack_weights(cfg)
    rng = np.random.default_rng(3)
    docs = [[rng.integers(1, cfg.vocab, size=int(rng.integers(5, 90))).tolist() for _ in range(4)]
            for _ in range(cfg.B)]
    sampler = txl.StreamSampler(docs, cfg.L, pad_id=0)
    st, keep = make_stack(cfg, w)
    emb = keep[0]
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    nll = torch.empty(cfg.B * cfg.L, dtype=torch.float32, device=DEV)
    o_tok, o_tgt, o_rst, _ = ev.row_streams(docs, cfg.L, cfg.n_seg, pad_id=0)
    worst = 0.0
    for s in range(cfg.n_seg):
        tok, tgt, rst, ln = sampler.next()
        assert (tok == o_tok[s]).all() and (tgt == o_tgt[s]).all() and (rst == o_rst[s]).all()
        if rst.any():
            txl.txl_mem_reset_rows(mems, torch.from_numpy(rst).to(DEV))
        st.step(torch.from_numpy(tok).to(DEV), mems, h)
        tg = torch.from_numpy(tgt.reshape(-1)).to(DEV)
        txl.txl_lm_loss(h.reshape(-1, cfg.d), emb, tg, nll)
        torch.cuda.synchronize()
        got = nll.cpu().double().numpy()
        ref = ev.segment_nll(f64(h.reshape(-1, cfg.d)), f64(emb), tgt.reshape(-1))
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        assert (err <= ATOL + RTOL * np.abs(ref)).all(), s
        assert (got[tgt.reshape(-1) < 0] == 0).all()
        # rows reset by the sampler start with no memory
        for m in mems[:-1]:
            v = m.valid.cpu().numpy()
            assert (v[rst.astype(bool)] == min(cfg.M, cfg.L)).all()
    say(f"evaluation stream: {cfg.n_seg} segments, max abs loss err {worst:.2e}")
    sampler.close()
    st.close()
    del keep
