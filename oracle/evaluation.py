"""fp64 oracle: stream sampling and the segment loss for evaluation.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

[P1] "Transformer-XL" notes:
  * "Stream Sampler Contract": every batch row is a state machine over its own
    stream of documents with state (doc_id, offset, reset). A step takes the
    next up to seg_len tokens of the current document; the flag returned is
    the one held before the step; reaching the end of the document moves the
    row to the next document (cyclically), back to offset 0, with the flag
    set, so that the next segment starts without context.
  * "Batched Streams": the reset flag is per row.
  * "Training Loop Sketch": the loss is the cross entropy of the current
    segment only.

Readings where the pages leave a step open (stated here and in the design
notes): the target of a token is the next token of the same document, so the
last token of a document has none; a segment shorter than seg_len (the end of
a document) is padded to seg_len with a pad id and its padded positions have
no target. Positions with no target carry target -1 and add nothing to the
loss.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _advance(state: dict, docs: Sequence[Sequence[int]], seg_len: int):
    """One step of a row's cursor {doc_id, offset, reset} over its documents:
    the next up to seg_len tokens of the current document, their next-token
    targets (-1 past the document's last token), and the flag the row held
    before the step. A row that reaches the end of its document moves to the
    next one (wrapping around) at offset 0 with the flag raised."""
    doc = docs[state["doc_id"]]
    lo = state["offset"]
    hi = len(doc) if lo + seg_len > len(doc) else lo + seg_len
    toks = [int(doc[p]) for p in range(lo, hi)]
    tgts = [int(doc[p + 1]) if p + 1 < len(doc) else -1 for p in range(lo, hi)]
    was_reset = state["reset"]
    if hi == len(doc):
        state.update(doc_id=(state["doc_id"] + 1) % len(docs), offset=0, reset=True)
    else:
        state.update(offset=hi, reset=False)
    return toks, tgts, was_reset


def row_streams(docs_per_row: Sequence[Sequence[Sequence[int]]], seg_len: int, n_seg: int,
                pad_id: int = 0):
    """Step one cursor per row n_seg times (every cursor starts at document 0,
    offset 0, flag raised). Returns int arrays tokens [n_seg, B, L] (padded
    with pad_id), targets [n_seg, B, L] (-1 for none), reset [n_seg, B] (0/1)
    and lengths [n_seg, B]."""
    B = len(docs_per_row)
    states = [{"doc_id": 0, "offset": 0, "reset": True} for _ in range(B)]
    tokens = np.full((n_seg, B, seg_len), pad_id, dtype=np.int64)
    targets = np.full((n_seg, B, seg_len), -1, dtype=np.int64)
    reset = np.zeros((n_seg, B), dtype=np.int64)
    lengths = np.zeros((n_seg, B), dtype=np.int64)
    for s in range(n_seg):
        for b in range(B):
            toks, tgts, rs = _advance(states[b], docs_per_row[b], seg_len)
            tokens[s, b, :len(toks)] = toks
            targets[s, b, :len(tgts)] = tgts
            reset[s, b] = int(rs)
            lengths[s, b] = len(toks)
    return tokens, targets, reset, lengths


def segment_nll(h: np.ndarray, w_out: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Per-token cross entropy of the current segment: for token n with
    logits z = w_out h_n (one per vocabulary entry),
    nll_n = log(sum_v exp(z_v)) - z_{target_n}, and 0 where target_n < 0.
    h [n, d], w_out [V, d], targets [n]; all in float64, one row at a time."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w_out, dtype=np.float64)
    out = np.zeros(h.shape[0])
    for n in range(h.shape[0]):
        t = int(targets[n])
        if t < 0:
            continue
        z = w @ h[n]
        zmax = z.max()
        lse = zmax + np.log(np.sum(np.exp(z - zmax)))
        out[n] = lse - z[t]
    return out
