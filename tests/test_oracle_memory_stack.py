"""Pins of the fp64 memory and stack oracle.

Memory: the FIFO closed form (after s segments from empty, memory is the last
min(M, s*L) states of the whole history). Stack: LayerNorm and GELU against
torch's fp64 routines, the sinusoid's internal properties, and the streaming
recurrence against a hand-unrolled rebuild of every layer's context from the
stored history.
"""
import math

import numpy as np
import pytest
import torch

from oracle import memory as om
from oracle import stack as ost


# ----------------------------------------------------------------------------
# memory
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,M", [(4, 8), (3, 3), (5, 2), (4, 0), (1, 7)])
def test_fifo_closed_form(L, M):
    """Tail_M of [mem; H] repeated s times from an empty memory leaves the
    last min(M, s*L) rows of the concatenated history ([P1] "Segment-Level
    Recurrence"; [P4] FIFO buffer)."""
    rng = np.random.default_rng(L * 10 + M)
    B, d = 2, 3
    mems = [np.zeros((B, 0, d)), np.zeros((B, 0, d))]
    hist = [np.zeros((B, 0, d)), np.zeros((B, 0, d))]
    for s in range(1, 6):
        hids = [rng.standard_normal((B, L, d)) for _ in range(2)]
        mems = om.update_mems(mems, hids, M)
        hist = [np.concatenate([a, h], axis=1) for a, h in zip(hist, hids)]
        keep = min(M, s * L)
        for m, hst in zip(mems, hist):
            assert m.shape == (B, keep, d)
            assert np.array_equal(m, hst[:, hst.shape[1] - keep:])


def test_zero_length_memory_keeps_nothing():
    h = [np.ones((2, 5, 3))]
    out = om.update_mems([np.ones((2, 4, 3))], h, 0)
    assert out[0].shape == (2, 0, 3)


def test_segment_longer_than_memory_keeps_last_rows():
    h = np.arange(2 * 6 * 1, dtype=float).reshape(2, 6, 1)
    out = om.update_mems([np.zeros((2, 4, 1))], [h], 4)[0]
    assert np.array_equal(out, h[:, 2:])


def test_update_rows_matches_batched_form():
    rng = np.random.default_rng(5)
    old = rng.standard_normal((3, 4, 2))
    h = rng.standard_normal((3, 3, 2))
    batched = om.update_mems([old], [h], 5)[0]
    rows = om.update_rows(list(old), h, 5)
    assert np.array_equal(np.stack(rows), batched)
    # a row with an empty memory (a reset) grows from nothing
    rows = om.update_rows([old[0], np.zeros((0, 2)), old[2]], h, 5)
    assert np.array_equal(rows[1], h[1])


# ----------------------------------------------------------------------------
# layer pieces
# ----------------------------------------------------------------------------
def test_layer_norm_matches_torch_fp64():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 32)) * 3 + 1
    g = rng.standard_normal(32)
    b = rng.standard_normal(32)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (32,),
                                         torch.from_numpy(g), torch.from_numpy(b),
                                         eps=ost.LN_EPS).numpy()
    np.testing.assert_allclose(ost.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)


def test_gelu_matches_torch_fp64():
    x = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(ost.gelu(x), ref, rtol=1e-13, atol=1e-15)


def test_sinusoid_properties():
    """Parity unpinned by the pages (they only say "sinusoidal"). The chosen
    form must still be a sinusoid of the distance: distance 0 gives
    [0..0 | 1..1], and inner products depend only on the difference of the
    distances (sum_k cos(f_k (a - b)))."""
    d = 16
    e0 = ost.sinusoid(np.array([0.0]), d)[0]
    assert np.array_equal(e0, np.r_[np.zeros(d // 2), np.ones(d // 2)])
    a = ost.sinusoid(np.array([3.0, 10.0, 7.0, 14.0]), d)
    np.testing.assert_allclose(a[0] @ a[1], a[2] @ a[3], rtol=1e-12)
    freq = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    np.testing.assert_allclose(a[0] @ a[1], np.cos(freq * 7.0).sum(), rtol=1e-12)


def test_rel_pos_table_row_order_and_heads():
    """Row t of R is the projected embedding of distance M+L-1-t; head h uses
    columns h*dh..(h+1)*dh-1 of W_R."""
    M, L, H, dh = 5, 3, 2, 4
    d = H * dh
    w = np.random.default_rng(2).standard_normal((d, H * dh))
    r = ost.rel_pos_table(w, M, L, H, dh)
    assert r.shape == (H, M + L, dh)
    for t in range(M + L):
        e = ost.sinusoid(np.array([M + L - 1 - t]), d)[0]
        for h in range(H):
            np.testing.assert_allclose(r[h, t], e @ w[:, h * dh:(h + 1) * dh],
                                       rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# the streamed stack
# ----------------------------------------------------------------------------
def _tiny_stack(seed=0, n_layer=2, d=16, H=2, dh=8, d_ff=24, vocab=40):
    rng = np.random.default_rng(seed)
    nrm = lambda *s: rng.standard_normal(s) * 0.3
    layers = []
    for _ in range(n_layer):
        layers.append({
            "wq": nrm(d, H * dh), "wk": nrm(d, H * dh), "wv": nrm(d, H * dh),
            "wo": nrm(H * dh, d), "wr": nrm(d, H * dh),
            "u": nrm(H, dh), "vb": nrm(H, dh),
            "w1": nrm(d, d_ff), "w2": nrm(d_ff, d),
            "ln1_g": 1 + nrm(d), "ln1_b": nrm(d), "ln2_g": 1 + nrm(d), "ln2_b": nrm(d),
        })
    emb = rng.standard_normal((vocab, d))
    return emb, layers


@pytest.mark.parametrize("L,M", [(3, 5), (4, 4), (5, 3)])
def test_stream_equals_unrolled_recurrence(L, M):
    """Streaming S segments through the per-layer memories equals rebuilding
    each layer's context by hand from the stored history: layer n at segment
    s reads the last M states of layer n-1 from the segments since the row's
    last reset, then the current H^(n-1) ([P1] "Segment-Level Recurrence";
    [P2] section 2, the dependency moving down one layer per segment)."""
    H, dh = 2, 8
    emb, layers = _tiny_stack()
    S, B = 6, 2
    rng = np.random.default_rng(9)
    tokens = rng.integers(0, emb.shape[0], (S, B, L))
    resets = np.zeros((S, B), dtype=np.uint8)
    resets[0] = 1
    resets[3, 1] = 1
    r_tables = [ost.rel_pos_table(lw["wr"], M, L, H, dh) for lw in layers]
    out = ost.stream(tokens, resets, emb, layers, r_tables, M, H, dh)
    for b in range(B):
        start = 0
        for s in range(S):
            if resets[s, b]:
                start = s
            h = emb[tokens[s, b]]
            for n, lw in enumerate(layers):
                hist = [out[p][b][n] for p in range(start, s)]
                past = np.concatenate(hist, axis=0) if hist else np.zeros((0, h.shape[1]))
                mem = past[max(0, past.shape[0] - M):]
                h = ost.layer_forward(h, mem, lw, r_tables[n], M, H, dh)
                np.testing.assert_array_equal(h, out[s][b][n + 1])


def test_reset_row_equals_fresh_stream():
    """A row that resets at segment s produces what a fresh stream started at
    segment s produces ([P1] "Stream Sampler Contract": memory is valid only
    while the row continues the same stream)."""
    H, dh, L, M = 2, 8, 3, 4
    emb, layers = _tiny_stack(seed=4)
    r_tables = [ost.rel_pos_table(lw["wr"], M, L, H, dh) for lw in layers]
    rng = np.random.default_rng(11)
    tokens = rng.integers(0, emb.shape[0], (5, 2, L))
    resets = np.zeros((5, 2), dtype=np.uint8)
    resets[0] = 1
    resets[2, 0] = 1
    full = ost.stream(tokens, resets, emb, layers, r_tables, M, H, dh)
    fresh = ost.stream(tokens[2:], resets[2:], emb, layers, r_tables, M, H, dh)
    for s in range(3):
        for n in range(len(layers) + 1):
            np.testing.assert_array_equal(full[s + 2][0][n], fresh[s][0][n])
    # row 1 did not reset, so it differs from a fresh start after segment 2
    assert not np.array_equal(full[2][1][2], fresh[0][1][2])


def test_first_segment_has_no_memory():
    H, dh, L, M = 2, 8, 3, 4
    emb, layers = _tiny_stack(seed=6)
    r_tables = [ost.rel_pos_table(lw["wr"], M, L, H, dh) for lw in layers]
    tokens = np.random.default_rng(1).integers(0, emb.shape[0], (1, 1, L))
    out = ost.stream(tokens, np.ones((1, 1)), emb, layers, r_tables, M, H, dh)
    h = emb[tokens[0, 0]]
    for n, lw in enumerate(layers):
        h = ost.layer_forward(h, np.zeros((0, 16)), lw, r_tables[n], M, H, dh)
        np.testing.assert_array_equal(h, out[0][0][n + 1])
    assert math.isfinite(float(out[0][0][-1].sum()))
