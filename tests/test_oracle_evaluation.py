"""Pins of the evaluation oracle (CPU): stream sampling and the segment loss.

The sampler follows [P1] "Stream Sampler Contract" (per-row state doc_id,
offset, reset; the next up to seg_len tokens of the current document; moving
to the next document at its end with reset raised). Its pins: an example
worked by hand from those rules, and invariants on random documents that any
correct reading must satisfy. The loss follows [P1] "Training Loop Sketch"
(cross entropy of the current segment); its pins: the closed form for
all-zero logits and PyTorch's fp64 cross entropy.
"""
import math

import numpy as np
import torch

from oracle import evaluation as ev


def test_sampler_hand_worked_example():
    """One row, documents A = 10 11 12 13 14 and B = 20 21, seg_len 3.
    Step 1 starts A (reset raised by construction): 10 11 12, targets 11 12 13.
    Step 2 continues A (no reset): 13 14 + pad, targets 14 and none (14 ends
    A), then the row moves to B. Step 3 starts B (reset): 20 21 + pad,
    targets 21 and none. Step 4 wraps around to A again (reset)."""
    t, g, r, n = ev.row_streams([[[10, 11, 12, 13, 14], [20, 21]]], 3, 5, pad_id=0)
    assert t[:, 0].tolist() == [[10, 11, 12], [13, 14, 0], [20, 21, 0], [10, 11, 12], [13, 14, 0]]
    assert g[:, 0].tolist() == [[11, 12, 13], [14, -1, -1], [21, -1, -1], [11, 12, 13], [14, -1, -1]]
    assert r[:, 0].tolist() == [1, 0, 1, 1, 0]
    assert n[:, 0].tolist() == [3, 2, 2, 3, 2]


def test_sampler_document_exactly_one_segment():
    """A document of exactly seg_len tokens is one segment; the next segment
    starts the following document with reset raised."""
    t, g, r, n = ev.row_streams([[[1, 2, 3], [4, 5, 6, 7]]], 3, 4)
    assert t[:, 0].tolist() == [[1, 2, 3], [4, 5, 6], [7, 0, 0], [1, 2, 3]]
    assert r[:, 0].tolist() == [1, 1, 0, 1]
    assert g[0, 0].tolist() == [2, 3, -1]


def random_docs(rng, B, n_docs, max_len, vocab):
    return [[rng.integers(1, vocab, size=int(rng.integers(1, max_len + 1))).tolist()
             for _ in range(n_docs)] for _ in range(B)]


def test_sampler_invariants_on_random_documents():
    rng = np.random.default_rng(0)
    B, L, n_seg = 5, 7, 60
    docs = random_docs(rng, B, 6, 30, 50)
    t, g, r, n = ev.row_streams(docs, L, n_seg, pad_id=0)
    for b in range(B):
        # segments between resets concatenate to the row's documents, in order
        pieces, cur = [], None
        for s in range(n_seg):
            seg = t[s, b, :n[s, b]].tolist()
            if r[s, b]:
                if cur is not None:
                    pieces.append(cur)
                cur = []
            cur += seg
            # padding only after the segment's tokens; no target there
            assert (t[s, b, n[s, b]:] == 0).all() and (g[s, b, n[s, b]:] == -1).all()
            assert 1 <= n[s, b] <= L
        k = 0
        for piece in pieces:          # every completed document, cyclically
            assert piece == docs[b][k % len(docs[b])]
            k += 1
        # a short segment always ends a document, so the next one resets
        for s in range(n_seg - 1):
            if n[s, b] < L:
                assert r[s + 1, b] == 1
        # targets: the next token of the same document
        for s in range(n_seg):
            for p in range(n[s, b] - 1):
                assert g[s, b, p] == t[s, b, p + 1]
            last = n[s, b] - 1
            if s + 1 < n_seg and not r[s + 1, b]:
                assert g[s, b, last] == t[s + 1, b, 0]
            elif s + 1 < n_seg:
                assert g[s, b, last] == -1


def test_nll_zero_logits_is_log_vocab():
    rng = np.random.default_rng(1)
    V, d, n = 37, 16, 9
    h = rng.standard_normal((n, d))
    tg = rng.integers(0, V, size=n)
    tg[3] = -1
    out = ev.segment_nll(h, np.zeros((V, d)), tg)
    want = np.full(n, math.log(V))
    want[3] = 0.0
    assert np.allclose(out, want, rtol=0, atol=1e-14)


def test_nll_matches_torch_cross_entropy_fp64():
    rng = np.random.default_rng(2)
    V, d, n = 101, 24, 40
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((V, d)) * 0.7
    tg = rng.integers(0, V, size=n)
    tg[::7] = -1
    out = ev.segment_nll(h, w, tg)
    logits = torch.from_numpy(h @ w.T)
    ref = torch.nn.functional.cross_entropy(logits, torch.from_numpy(tg), ignore_index=-1,
                                            reduction="none").numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-12)


def test_nll_large_logit_limit():
    """A target logit far above the others gives a loss near 0; far below, a
    loss near the gap."""
    d, V = 4, 6
    h = np.array([[1.0, 0, 0, 0]])
    w = np.zeros((V, d))
    w[2, 0] = 60.0
    assert ev.segment_nll(h, w, np.array([2]))[0] < 1e-20
    assert abs(ev.segment_nll(h, w, np.array([0]))[0] - 60.0) < 1e-12
