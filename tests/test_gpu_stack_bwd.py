"""GPU parity of the stack's training step (txl_segment_step_train) and its
segment gradients (txl_segment_backward) against the fp64 oracle
(oracle/stack.py segment_backward_row, pinned by finite differences).

The oracle runs the whole segment in fp64 from the same token ids, weights
and memories (the rings as the GPU held them before the step), and takes the
gradient dy at the top; a batch's weight gradient is the sum of its rows'.
Memory slots a row does not hold are filled with NaN on the GPU: they must
not reach any gradient.

Tolerance, per gradient tensor, normwise: ||gpu - ref|| <= TOL ||ref||.
Every product of the backward takes bf16 operands (activations of the
tape, dX, dFpre, dA, the packed dQ / dK / dV, the attention's P and dS)
with fp32 accumulation, so each operand carries a relative rounding error
of at most 2^-9 (rms 2^-9 / sqrt(3) = 1.1e-3), independent between
roundings. A weight gradient is reached through about 20 such roundings
along its longest path (forward and backward of two layers), which adds up
in quadrature to about sqrt(20) * 1.1e-3 = 5e-3 relative; TOL = 2e-2 leaves
a factor 4 (measured: at most 9e-3 on the two-layer stacks, 6e-3 on every
layer of the sixteen-layer one). The attention's D_i = dout_i . out_i is
formed from the forward's unrounded output: from the bf16 output, its
rounding came back magnified in the score-path gradients of deep layers
(W_R, v, W^Q, W^K up to 2.3e-2 at layer 16), which a CPU replay of the
oracle with out rounded in D alone reproduces. Rows of the embedding
gradient for tokens absent from the segment must be exactly 0, and two
calls must give identical bits.
"""
import dataclasses

import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import stack as ost
from tests.gpu_helpers import f64, say
from tests.test_gpu_stack import make_stack, read_rings, OUT_MAJOR

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def _cfg(**kw):
    base = dict(n_layer=2, d=256, H=4, d_h=64, d_ff=512, vocab=97, B=3, L=40, M=72, n_seg=3,
                seed=5, w_std=0.05, reset_every=0)
    base.update(kw)
    return txl_synth.StackConfig("bwd", "bf16", **base)


def _rings(cfg):
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    for m in mems:
        m.data.fill_(float("nan"))       # slots never written stay NaN
    return mems


def _train_step(cfg, w, warm_resets):
    """Stream segments 0 .. n_seg-2 (resets before each as given), then the
    training step on segment n_seg-1. Returns the stack, the tape, the rings
    before and after the training step (fp64 logical, valid) and the
    step's tokens."""
    st, keep = make_stack(cfg, w)
    mems = _rings(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    h_out = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    tok_d = tokens.to(DEV)
    for s in range(cfg.n_seg):
        if warm_resets[s].any():
            txl.txl_mem_reset_rows(mems, warm_resets[s].to(DEV).contiguous())
        if s + 1 < cfg.n_seg:
            st.step(tok_d[s].contiguous(), mems, h_out)
    before = read_rings(mems)
    tape = st.new_tape()
    st.step_train(tok_d[cfg.n_seg - 1].contiguous(), mems, h_out, tape)
    torch.cuda.synchronize()
    after = read_rings(mems)
    return st, keep, tape, before, after, tokens[cfg.n_seg - 1].numpy()


def _oracle_grads(cfg, w, before, tokens, dy, rows):
    """Sum over batch rows `rows` of the oracle's segment gradients."""
    emb = f64(w["emb"])
    layers = [{k: f64(t) for k, t in lw.items()} for lw in w["layers"]]
    demb = np.zeros_like(emb)
    acc = None
    for b in rows:
        mems = [before[n][0][b, cfg.M - before[n][1][b]:] for n in range(cfg.n_layer + 1)]
        de, g = ost.segment_backward_row(tokens[b], mems, emb, layers, cfg.M, cfg.H, cfg.d_h,
                                         dy[b])
        demb += de
        if acc is None:
            acc = g
        else:
            for n in range(cfg.n_layer):
                for k in acc[n]:
                    acc[n][k] = acc[n][k] + g[n][k]
    return demb, acc


def _oracle_grads_forced(cfg, w, before, after, tokens, dy, b):
    """One batch row, teacher-forced: layer n (from the top down) gets the
    GPU's own bf16 input H^(n-1) (the last L rows of ring n-1 after the
    step; needs L <= M) and its memory before the step, and the oracle's
    fp64 gradient from the layer above. The GPU's forward rounding then
    stays out of the comparison, as in the forward parity tests."""
    emb = f64(w["emb"])
    M, L = cfg.M, cfg.L
    assert L <= M
    g_h = np.asarray(dy[b], dtype=np.float64)
    grads = [None] * cfg.n_layer
    for n in range(cfg.n_layer - 1, -1, -1):
        lw = {k: f64(t) for k, t in w["layers"][n].items()}
        h_in = after[n][0][b, M - L:]
        mem = before[n][0][b, M - before[n][1][b]:]
        g_h, grads[n] = ost.layer_backward(h_in, mem, lw, lw["wr"], M, cfg.H, cfg.d_h, g_h)
    demb = np.zeros_like(emb)
    for pos, t in enumerate(tokens[b]):
        demb[t] += g_h[pos]
    return demb, grads


def _gpu_in_oracle_layout(grads):
    emb = f64(grads["emb"])
    layers = []
    for lg in grads["layers"]:
        layers.append({k: (f64(t).T if k in OUT_MAJOR else f64(t)) for k, t in lg.items()})
    return emb, layers


def _compare(cfg, got, want, tokens, what):
    g_emb, g_layers = got
    w_emb, w_layers = want
    worst, over = 0.0, []
    for n in range(cfg.n_layer):
        for k in sorted(w_layers[n]):
            a, b = g_layers[n][k], w_layers[n][k]
            assert a.shape == b.shape, (n, k, a.shape, b.shape)
            assert np.isfinite(a).all(), (what, n, k)
            rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
            worst = max(worst, rel)
            say(f"  {what} layer {n + 1} {k:6s}: normwise rel err {rel:.2e}")
            if rel > TOL:
                over.append((n + 1, k, rel))
    assert not over, (what, over)
    present = np.zeros(cfg.vocab, dtype=bool)
    present[np.asarray(tokens).reshape(-1)] = True
    assert np.isfinite(g_emb).all()
    assert np.abs(g_emb[~present]).max(initial=0.0) == 0.0
    rel = float(np.linalg.norm(g_emb - w_emb) / np.linalg.norm(w_emb))
    say(f"  {what} emb: normwise rel err {rel:.2e} over {int(present.sum())} present tokens")
    assert rel <= TOL
    return max(worst, rel)


def test_training_step_forward_equals_inference_step_bitwise():
    """The recording step computes what txl_segment_step computes."""
    cfg = _cfg()
    w = txl_synth.stack_weights(cfg, ln_std=0.1)
    st, keep = make_stack(cfg, w)
    tokens = txl_synth.stack_tokens(cfg).to(DEV)
    a, b = _rings(cfg), _rings(cfg)
    ha = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    hb = torch.empty_like(ha)
    tape = st.new_tape()
    for s in range(cfg.n_seg):
        st.step(tokens[s].contiguous(), a, ha)
        st.step_train(tokens[s].contiguous(), b, hb, tape)
        torch.cuda.synchronize()
        assert torch.equal(ha, hb), s
        for ra, rb in zip(read_rings(a), read_rings(b)):
            assert np.array_equal(ra[1], rb[1])
            for row in range(cfg.B):
                v = ra[1][row]
                assert np.array_equal(ra[0][row, cfg.M - v:], rb[0][row, cfg.M - v:])
    st.close()
    del keep


@pytest.mark.parametrize("case", ["mixed_memory", "no_memory_ragged"])
def test_segment_gradients_match_oracle(case):
    """Two layers; rows with a partial memory, a full one and none (reset
    just before the step), or M = 0 with a ragged L (50 rows per batch row:
    the padded reductions end in a partial tile)."""
    if case == "mixed_memory":
        # M + L = 240 keys: the attention runs in two key splits
        cfg = _cfg(M=200, n_seg=7)
        resets = txl_synth.reset_schedule(cfg)
        resets[5, 0] = 1                  # row 0: one segment of memory (40 of 200)
        resets[6, 2] = 1                  # row 2: no memory at the training step
                                          # row 1: a full, wrapped ring
    else:
        cfg = _cfg(M=0, L=50, B=2, n_seg=2, seed=8)
        resets = txl_synth.reset_schedule(cfg)
    w = txl_synth.stack_weights(cfg, ln_std=0.1)
    st, keep, tape, before, _, tokens = _train_step(cfg, w, resets)
    say(f"{case}: valid before the step {[int(v) for v in before[0][1]]}")
    dy = txl_synth.stack_dy(cfg)
    grads = st.new_grads()
    st.backward(tape, dy.to(DEV).contiguous(), grads)
    torch.cuda.synchronize()
    got = _gpu_in_oracle_layout(grads)
    want = _oracle_grads(cfg, w, before, tokens, dy.double().numpy(), range(cfg.B))
    _compare(cfg, got, want, tokens, case)
    # deterministic: a second call gives the same bits
    again = st.new_grads()
    st.backward(tape, dy.to(DEV).contiguous(), again)
    torch.cuda.synchronize()
    assert torch.equal(grads["emb"], again["emb"])
    for lg, la in zip(grads["layers"], again["layers"]):
        for k in lg:
            assert torch.equal(lg[k], la[k]), k
    st.close()
    del keep


@pytest.mark.timeout(600)
def test_sixteen_layers_full_size_one_row():
    """The 16-layer d=512 stack at its full size (B=16, L=384, M=384), in the
    launch configuration of the full batch. Batch rows do not interact, so
    with dy zero on every row but one the weight gradients are that row's
    alone, which the oracle computes for all sixteen layers."""
    cfg = txl_synth.STACK_CONFIGS["16layer_d512"]
    cfg = dataclasses.replace(cfg, n_seg=2)
    w = txl_synth.stack_weights(cfg, ln_std=0.1)
    resets = txl_synth.reset_schedule(cfg)
    st, keep, tape, before, after, tokens = _train_step(cfg, w, resets)
    row = 5
    dy = txl_synth.stack_dy(cfg)
    dy[:row] = 0
    dy[row + 1:] = 0
    grads = st.new_grads()
    st.backward(tape, dy.to(DEV).contiguous(), grads)
    torch.cuda.synchronize()
    got = _gpu_in_oracle_layout(grads)
    say(f"full size: memory of row {row} holds {int(before[0][1][row])} slots; oracle running")
    want = _oracle_grads_forced(cfg, w, before, after, tokens, dy.double().numpy(), row)
    _compare(cfg, got, want, tokens[row:row + 1], "16-layer row 5")
    st.close()
    del keep
