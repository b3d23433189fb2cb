"""fp64 oracle: the per-layer FIFO memory, as plain variable-length arrays.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

[P1] "Transformer-XL" notes, section "Segment-Level Recurrence": after the
step, each layer's memory becomes Tail_M([M; H]), the last M hidden states of
the old memory followed by the current segment. Section "Batched Tensor
Contract" gives the batched contract: concatenate along the sequence axis,
keep the last mem_len rows (all of them when fewer), and keep nothing when
mem_len is 0. [P4] "Transformer-XL" describes the same thing as a FIFO buffer
that overwrites its oldest entries.

The oracle keeps memory as ordinary arrays whose length grows until it
reaches M: there is no ring, no head pointer and no valid counter.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def tail(x: np.ndarray, m: int, axis: int = 0) -> np.ndarray:
    """Tail_m along ``axis``: the last m entries, or all when fewer; m = 0 -> empty."""
    n = x.shape[axis]
    if m == 0:
        return np.take(x, np.arange(0), axis=axis)
    return np.take(x, np.arange(max(0, n - m), n), axis=axis)


def update_mems(mems: Sequence[np.ndarray], hids: Sequence[np.ndarray],
                mem_len: int) -> List[np.ndarray]:
    """Batched update of every layer's memory (arrays [B, m, d] and [B, L, d]).

    Returns new arrays (copies: the detach of the page is a copy here, the
    oracle has no autograd). mem_len == 0 keeps an empty memory.
    """
    out = []
    for old, cur in zip(mems, hids):
        cat = np.concatenate([np.asarray(old, dtype=np.float64),
                              np.asarray(cur, dtype=np.float64)], axis=1)
        out.append(tail(cat, mem_len, axis=1).copy())
    return out


def update_rows(mem_rows: Sequence[np.ndarray], h: np.ndarray, mem_len: int
                ) -> List[np.ndarray]:
    """Per-row form of the update for rows whose memories differ in length
    (rows that reset at a document boundary, [P1] section "Batched Streams"):
    row b's memory [m_b, d] becomes Tail_mem_len([mem_b; h_b])."""
    return [tail(np.concatenate([np.asarray(m, dtype=np.float64),
                                 np.asarray(hb, dtype=np.float64)], axis=0),
                 mem_len, axis=0).copy()
            for m, hb in zip(mem_rows, h)]
