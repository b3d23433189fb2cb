"""Pins of the oracle's layer composition (oracle/stack.py ``layer_forward``).

The pages fix Q from the current segment and K, V from [SG(mem); H]; the rest
of the layer (W^O, post-LayerNorm, GELU feed-forward) is a stated reading.
These tests tie the composition to things other than itself:

* with the two sublayers switched off (W^O = 0, W2 = 0) a layer is two
  LayerNorms of its input, computed here with torch's fp64 layer_norm;
* with one head, identity projections, u = v = 0 and W_R = 0 the attention
  sublayer is standard softmax attention of the segment over [memory;
  segment] under the rectangular mask, computed with torch's fp64
  scaled_dot_product_attention (independent of the oracle's attention);
* the same with u, v and W_R switched on at a full memory equals the oracle's
  pinned attention on the raw states (Q from h, K/V from [mem; h], memory
  first);
* a memory of m <= M stored states reads the last m + L rows of a
  capacity-M table: the call with the capacity-M table equals the call with
  a table built for capacity m, for every m;
* permuting the heads (their column blocks of W^Q, W^K, W^V, W_R, the rows
  of u and v, and the matching row blocks of W^O) leaves the output
  unchanged;
* the weights' orientation: d differs from H*d_h, so a transposed product
  cannot run.

Every pin is then run against the oracle with one step replaced by a
plausible mistake (swapped LayerNorm parameters, pre-LN order, the first
m + L rows of R, a head split that takes every H-th column, K/V with the
memory last) and must fail there.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import stack as ost

L_, M_, H_, DH_, D_, DFF_ = 5, 7, 2, 4, 12, 10   # d = 12 differs from H*d_h = 8


def _weights(seed, d=D_, H=H_, dh=DH_, d_ff=DFF_):
    rng = np.random.default_rng(seed)
    nrm = lambda *s: rng.standard_normal(s) * 0.4
    return {
        "wq": nrm(d, H * dh), "wk": nrm(d, H * dh), "wv": nrm(d, H * dh),
        "wo": nrm(H * dh, d), "wr": nrm(d, H * dh),
        "u": nrm(H, dh), "vb": nrm(H, dh),
        "w1": nrm(d, d_ff), "w2": nrm(d_ff, d),
        "ln1_g": 1 + nrm(d), "ln1_b": nrm(d), "ln2_g": 1 + nrm(d), "ln2_b": nrm(d),
    }


def _states(seed, n, d=D_):
    return np.random.default_rng(seed).standard_normal((n, d))


def _torch_ln(x, g, b):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.layer_norm(t(x), (x.shape[-1],), t(g), t(b),
                                          eps=ost.LN_EPS).numpy()


# ----------------------------------------------------------------------------
# the pins, as functions so that the planted-mistake tests can run them too
# ----------------------------------------------------------------------------
def pin_two_layernorms():
    """W^O = 0 and W2 = 0: the layer is LN2(LN1(h)) (torch fp64 layer_norm)."""
    lw = _weights(1)
    lw["wo"] = np.zeros_like(lw["wo"])
    lw["w2"] = np.zeros_like(lw["w2"])
    h = _states(2, L_) * 3 + 1
    mem = _states(3, M_)
    r = ost.rel_pos_table(lw["wr"], M_, L_, H_, DH_)
    got = ost.layer_forward(h, mem, lw, r, M_, H_, DH_)
    ref = _torch_ln(_torch_ln(h, lw["ln1_g"], lw["ln1_b"]), lw["ln2_g"], lw["ln2_b"])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _one_head_identity(seed, m):
    """One head, d = d_h, identity Q/K/V/O projections, W1 = 0 (so the
    feed-forward adds nothing), unit LayerNorms."""
    dh = 6
    lw = _weights(seed, d=dh, H=1, dh=dh, d_ff=7)
    eye = np.eye(dh)
    lw.update(wq=eye, wk=eye, wv=eye, wo=eye, w1=np.zeros((dh, 7)))
    for n in ("ln1_g", "ln2_g"):
        lw[n] = np.ones(dh)
    for n in ("ln1_b", "ln2_b"):
        lw[n] = np.zeros(dh)
    h = _states(seed + 1, L_, dh)
    mem = _states(seed + 2, m, dh)
    return lw, h, mem, dh


def pin_attention_sublayer_is_masked_sdpa():
    """u = v = 0, W_R = 0: the attention sublayer is softmax attention of
    the segment's states over [memory; segment] with the memory block
    visible and the segment block causal (torch fp64 SDPA); the layer is then
    LN(LN(h + A)) with unit LayerNorms."""
    for m in (0, 3, M_):
        lw, h, mem, dh = _one_head_identity(11, m)
        lw["u"] = np.zeros_like(lw["u"])
        lw["vb"] = np.zeros_like(lw["vb"])
        lw["wr"] = np.zeros_like(lw["wr"])
        r = ost.rel_pos_table(lw["wr"], M_, L_, 1, dh)
        got = ost.layer_forward(h, mem, lw, r, M_, 1, dh)
        keys = np.concatenate([mem, h], axis=0)
        visible = np.zeros((L_, m + L_), dtype=bool)
        visible[:, :m] = True
        visible[:, m:] = np.tril(np.ones((L_, L_), dtype=bool))
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
        att = torch.nn.functional.scaled_dot_product_attention(
            t(h[None]), t(keys[None]), t(keys[None]), attn_mask=t(visible[None]),
            scale=1.0 / math.sqrt(dh)).numpy()[0]
        one, zero = np.ones(dh), np.zeros(dh)
        ref = _torch_ln(_torch_ln(h + att, one, zero), one, zero)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def pin_attention_sublayer_is_rel_attn_on_raw_states():
    """u, v, W_R switched on, memory full (the whole table in use): the
    attention sublayer equals the oracle's pinned relative attention with
    q = h and k = v = [mem; h]."""
    lw, h, mem, dh = _one_head_identity(21, M_)
    r = ost.rel_pos_table(lw["wr"], M_, L_, 1, dh)
    got = ost.layer_forward(h, mem, lw, r, M_, 1, dh)
    keys = np.concatenate([mem, h], axis=0)
    att = oa.rel_attn(h[None, None], keys[None, None], keys[None, None], r,
                      lw["u"], lw["vb"], valid=[M_])["out"][0, 0]
    one, zero = np.ones(dh), np.zeros(dh)
    ref = _torch_ln(_torch_ln(h + att, one, zero), one, zero)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def pin_partial_memory_reads_last_rows():
    """A memory of m stored states under a capacity-M table gives exactly
    what the table built for capacity m gives, for every m <= M."""
    lw = _weights(31)
    h = _states(32, L_)
    mem_all = _states(33, M_)
    r_full = ost.rel_pos_table(lw["wr"], M_, L_, H_, DH_)
    for m in range(M_ + 1):
        mem = mem_all[M_ - m:]
        r_m = ost.rel_pos_table(lw["wr"], m, L_, H_, DH_)
        a = ost.layer_forward(h, mem, lw, r_full, M_, H_, DH_)
        b = ost.layer_forward(h, mem, lw, r_m, m, H_, DH_)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def pin_head_permutation():
    """Relabelling the heads (column blocks of W^Q, W^K, W^V, W_R, rows of
    u and v, row blocks of W^O) leaves the layer's output unchanged."""
    H, dh = 3, 4
    lw = _weights(41, H=H, dh=dh)
    h = _states(42, L_)
    mem = _states(43, 4)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * dh, (p + 1) * dh) for p in perm])
    pw = dict(lw)
    for n in ("wq", "wk", "wv", "wr"):
        pw[n] = lw[n][:, cols]
    pw["wo"] = lw["wo"][cols, :]
    pw["u"] = lw["u"][perm]
    pw["vb"] = lw["vb"][perm]
    r = ost.rel_pos_table(lw["wr"], M_, L_, H, dh)
    rp = ost.rel_pos_table(pw["wr"], M_, L_, H, dh)
    a = ost.layer_forward(h, mem, lw, r, M_, H, dh)
    b = ost.layer_forward(h, mem, pw, rp, M_, H, dh)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # and the heads are not interchangeable without moving W^O's blocks
    pw["wo"] = lw["wo"]
    c = ost.layer_forward(h, mem, pw, rp, M_, H, dh)
    assert np.abs(c - a).max() > 1e-3


PINS = [pin_two_layernorms, pin_attention_sublayer_is_masked_sdpa,
        pin_attention_sublayer_is_rel_attn_on_raw_states,
        pin_partial_memory_reads_last_rows, pin_head_permutation]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_layer_pin(pin):
    pin()


def test_split_and_merge_heads_are_column_blocks():
    x = np.arange(3 * 8, dtype=float).reshape(3, 8)
    s = ost.split_heads(x, 2, 4)
    assert np.array_equal(s[0], x[:, :4]) and np.array_equal(s[1], x[:, 4:])
    assert np.array_equal(ost.merge_heads(s), x)


def test_weight_orientation_is_input_by_output():
    """d = 12 and H*d_h = 8 differ, so x W with W stored [in, out] is the
    only product that runs; the output has the model width."""
    lw = _weights(51)
    r = ost.rel_pos_table(lw["wr"], M_, L_, H_, DH_)
    out = ost.layer_forward(_states(52, L_), _states(53, M_), lw, r, M_, H_, DH_)
    assert out.shape == (L_, D_)
    bad = dict(lw)
    bad["wq"] = lw["wq"].T
    with pytest.raises(ValueError):
        ost.layer_forward(_states(52, L_), _states(53, M_), bad, r, M_, H_, DH_)


# ----------------------------------------------------------------------------
# planted mistakes (in the oracle, on the CPU): each pin must catch its kind
# ----------------------------------------------------------------------------
def _swapped_ln_weights(w):
    """The layer's weights with LN1's and LN2's gains and shifts exchanged."""
    out = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    for a, b in (("ln1_g", "ln2_g"), ("ln1_b", "ln2_b")):
        out[a], out[b] = out[b], out[a]
    return out


def _pre_ln(x, f, g, b):
    return x + f          # residual without the normalisation


def _first_rows(r_table, M, m):
    r_table = np.asarray(r_table, dtype=np.float64)
    L = r_table.shape[1] - M
    return r_table[:, : m + L, :]


def _strided_heads(x, H, dh):
    n = x.shape[0]
    return x.reshape(n, dh, H).transpose(2, 0, 1).copy()


MISTAKES = {
    "layernorm parameters swapped": ("_f64", _swapped_ln_weights, [pin_two_layernorms]),
    "post-LN dropped (pre-LN residual)": ("add_norm", _pre_ln,
                                          [pin_two_layernorms,
                                           pin_attention_sublayer_is_masked_sdpa]),
    "first m+L rows of R": ("r_for_memory", _first_rows, [pin_partial_memory_reads_last_rows]),
    "head split takes every H-th column": ("split_heads", _strided_heads, [pin_head_permutation]),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, repl, pins = MISTAKES[name]
    monkeypatch.setattr(ost, attr, repl)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


def test_pin_catches_memory_last(monkeypatch):
    """K/V built from [h; mem] instead of [mem; h]: the masked-SDPA pin and
    the relative-attention pin both fail."""
    monkeypatch.setattr(ost, "context", lambda mem, h: np.concatenate([h, mem], axis=0))
    for pin in (pin_attention_sublayer_is_masked_sdpa,
                pin_attention_sublayer_is_rel_attn_on_raw_states):
        with pytest.raises(AssertionError):
            pin()
