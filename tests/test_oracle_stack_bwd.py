"""Pins of the oracle's segment gradients (oracle/stack.py layer_backward,
segment_backward_row) by central finite differences of the pinned forward.

The loss is sum(dy * out) for a fixed random dy, so its derivative with
respect to any parameter is what the backward returns for it. Every entry of
every weight of a tiny layer is checked (W^Q, W^K, W^V, W^O, W_R through the
relative-position table, u, v, both LayerNorms, both feed-forward matrices),
and the segment input; the memory is a stop-gradient input, held fixed, and
its rows must still feed W^K and W^V. A planted mistake in the LayerNorm or
GELU derivative fails the check.
"""
import numpy as np
import pytest

from oracle import stack as ost

L_, M_, H_, DH_, D_, DFF_ = 3, 4, 2, 2, 6, 5
EPS = 1e-6


def _layer(seed, d=D_, H=H_, dh=DH_, d_ff=DFF_):
    rng = np.random.default_rng(seed)
    nrm = lambda *s: rng.standard_normal(s) * 0.6
    return {
        "wq": nrm(d, H * dh), "wk": nrm(d, H * dh), "wv": nrm(d, H * dh),
        "wo": nrm(H * dh, d), "wr": nrm(d, H * dh),
        "u": nrm(H, dh), "vb": nrm(H, dh),
        "w1": nrm(d, d_ff), "w2": nrm(d_ff, d),
        "ln1_g": 1 + nrm(d), "ln1_b": nrm(d), "ln2_g": 1 + nrm(d), "ln2_b": nrm(d),
    }


def _loss(h, mem, lw, dy):
    r = ost.rel_pos_table(lw["wr"], M_, L_, H_, DH_)
    return float((dy * ost.layer_forward(h, mem, lw, r, M_, H_, DH_)).sum())


def _fd(f, x):
    """Central differences of the scalar f() with respect to every entry of
    the array x (perturbed in place)."""
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + EPS
        up = f()
        x[idx] = keep - EPS
        dn = f()
        x[idx] = keep
        g[idx] = (up - dn) / (2 * EPS)
    return g


def _check(got, want, what):
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got - want).max())
    assert err <= 1e-6 * scale, (what, err, scale)


def _case(m, seed=1):
    lw = _layer(seed)
    rng = np.random.default_rng(seed + 100)
    h = rng.standard_normal((L_, D_))
    mem = rng.standard_normal((M_, D_))[M_ - m:]
    dy = rng.standard_normal((L_, D_))
    return lw, h, mem, dy


@pytest.mark.parametrize("m", [0, 3, M_])
def test_layer_backward_every_weight_by_finite_differences(m):
    lw, h, mem, dy = _case(m)
    _, grads = ost.layer_backward(h, mem, lw, lw["wr"], M_, H_, DH_, dy)
    for name in sorted(lw):
        fd = _fd(lambda: _loss(h, mem, lw, dy), lw[name])
        _check(grads[name], fd, f"{name} (memory of {m})")


@pytest.mark.parametrize("m", [0, M_])
def test_layer_backward_input_by_finite_differences(m):
    lw, h, mem, dy = _case(m, seed=7)
    dh, _ = ost.layer_backward(h, mem, lw, lw["wr"], M_, H_, DH_, dy)
    _check(dh, _fd(lambda: _loss(h, mem, lw, dy), h), "h")


def test_memory_is_a_stop_gradient_input_that_still_feeds_wk_wv():
    """The forward depends on the memory (its finite-difference derivative
    is not zero), the backward returns nothing for it, and the memory rows
    change the W^K / W^V gradients (the finite differences above include
    them, with the memory held fixed)."""
    lw, h, mem, dy = _case(M_, seed=3)
    assert np.abs(_fd(lambda: _loss(h, mem, lw, dy), mem)).max() > 1e-3
    out = ost.layer_backward(h, mem, lw, lw["wr"], M_, H_, DH_, dy)
    assert len(out) == 2                         # (dh of the segment, weight grads)
    _, with_mem = out
    _, no_mem = ost.layer_backward(h, mem[:0], lw, lw["wr"], M_, H_, DH_, dy)
    assert np.abs(with_mem["wk"] - no_mem["wk"]).max() > 1e-3
    assert np.abs(with_mem["wv"] - no_mem["wv"]).max() > 1e-3


def test_segment_backward_embedding_and_first_layer():
    """Two layers, a repeated token: the gradient of sum(dy * H^(2)) with
    respect to the embedding rows and to the first layer's W^Q and W_R."""
    rng = np.random.default_rng(11)
    layers = [_layer(21), _layer(22)]
    vocab = 7
    emb = rng.standard_normal((vocab, D_))
    tokens = np.array([2, 5, 2])                 # token 2 twice
    mems = [rng.standard_normal((2, D_)), rng.standard_normal((2, D_)), np.zeros((0, D_))]
    dy = rng.standard_normal((L_, D_))

    def loss():
        r = [ost.rel_pos_table(lw["wr"], M_, L_, H_, DH_) for lw in layers]
        hs, _ = ost.segment_step_row(tokens, mems, emb, layers, r, M_, H_, DH_)
        return float((dy * hs[-1]).sum())

    demb, grads = ost.segment_backward_row(tokens, mems, emb, layers, M_, H_, DH_, dy)
    _check(demb, _fd(loss, emb), "emb")
    assert np.abs(demb[[0, 1, 3, 4, 6]]).max() == 0.0          # unused rows
    _check(grads[0]["wq"], _fd(loss, layers[0]["wq"]), "layer 1 wq")
    _check(grads[0]["wr"], _fd(loss, layers[0]["wr"]), "layer 1 wr")
    _check(grads[1]["w2"], _fd(loss, layers[1]["w2"]), "layer 2 w2")


def test_layer_norm_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 9)) * 2 + 0.5
    g = rng.standard_normal(9)
    b = rng.standard_normal(9)
    dy = rng.standard_normal((4, 9))
    dx, dg, db = ost.layer_norm_backward(x, g, dy)
    f = lambda: float((dy * ost.layer_norm(x, g, b)).sum())
    _check(dx, _fd(f, x), "dx")
    _check(dg, _fd(f, g), "dg")
    _check(db, _fd(f, b), "db")


def test_gelu_grad_matches_finite_differences():
    x = np.linspace(-6, 6, 241)
    fd = (ost.gelu(x + EPS) - ost.gelu(x - EPS)) / (2 * EPS)
    np.testing.assert_allclose(ost.gelu_grad(x), fd, rtol=1e-7, atol=1e-9)


# planted mistakes (in the oracle, on the CPU)
def _ln_bwd_no_xhat_term(x, g, dy, eps=ost.LN_EPS):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xhat = (x - mu) * r
    gdy = dy * g
    return r * (gdy - gdy.mean(axis=-1, keepdims=True)), (dy * xhat).sum(axis=0), dy.sum(axis=0)


@pytest.mark.parametrize("attr,mutant", [
    ("layer_norm_backward", _ln_bwd_no_xhat_term),
    ("gelu_grad", lambda x: 0.5 * (1.0 + np.tanh(x))),
])
def test_planted_mistake_fails_the_check(attr, mutant, monkeypatch):
    lw, h, mem, dy = _case(M_, seed=9)
    monkeypatch.setattr(ost, attr, mutant)
    dh, grads = ost.layer_backward(h, mem, lw, lw["wr"], M_, H_, DH_, dy)
    monkeypatch.undo()
    with pytest.raises(AssertionError):
        _check(grads["w1"], _fd(lambda: _loss(h, mem, lw, dy), lw["w1"]), "w1")
        _check(dh, _fd(lambda: _loss(h, mem, lw, dy), h), "h")
