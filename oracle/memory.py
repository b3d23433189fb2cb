"""fp64 oracle: the per-layer FIFO memory, as plain variable-length arrays.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

[P1] "Transformer-XL" notes, section "Segment-Level Recurrence": after the
step, each layer's memory becomes Tail_M([M; H]), the last M hidden states of
the old memory followed by the current segment. Section "Batched Tensor
Contract" states the batched contract in words: join memory and segment along
the sequence axis, keep the last mem_len rows (all of them when there are
fewer), keep nothing when mem_len is 0. [P4] "Transformer-XL" describes the
same thing as a FIFO buffer that overwrites its oldest entries.

The oracle keeps memory as ordinary arrays whose length grows until it
reaches M: there is no ring, no head pointer and no valid counter. Tail_M is
written as index arithmetic on the joined sequence: with n_old memory rows
and L segment rows the joined sequence has n = n_old + L rows, of which the
last keep = min(M, n) survive; surviving row k is joined row c = n - keep + k,
which is memory row c when c < n_old and segment row c - n_old otherwise.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def tail_rows(old: np.ndarray, cur: np.ndarray, m: int) -> np.ndarray:
    """Tail_m([old; cur]) for one row's memory old [n_old, ...] and segment
    cur [L, ...]: the last m rows of the joined sequence (all of them when
    fewer; none when m = 0), by index, never materialising the join."""
    old = np.asarray(old, dtype=np.float64)
    cur = np.asarray(cur, dtype=np.float64)
    n_old = old.shape[0]
    n = n_old + cur.shape[0]
    keep = min(m, n)
    out = np.empty((keep,) + cur.shape[1:])
    for k in range(keep):
        c = n - keep + k
        out[k] = old[c] if c < n_old else cur[c - n_old]
    return out


def tail(x: np.ndarray, m: int, axis: int = 0) -> np.ndarray:
    """Tail_m of one sequence along ``axis``: its last m entries, all of them
    when fewer, none when m = 0 (the join of nothing with x)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, 0)
    out = tail_rows(np.zeros((0,) + x.shape[1:]), x, m)
    return np.moveaxis(out, 0, axis)


def update_mems(mems: Sequence[np.ndarray], hids: Sequence[np.ndarray],
                mem_len: int) -> List[np.ndarray]:
    """Batched update of every layer's memory (arrays [B, m, d] and [B, L, d]).

    Returns new arrays (the detach of the page is a copy here, the oracle has
    no autograd): layer by layer and batch row by batch row, Tail_mem_len of
    the memory followed by the segment. mem_len == 0 keeps an empty memory.
    """
    out = []
    for old, cur in zip(mems, hids):
        old = np.asarray(old, dtype=np.float64)
        cur = np.asarray(cur, dtype=np.float64)
        rows = [tail_rows(old[b], cur[b], mem_len) for b in range(cur.shape[0])]
        keep = min(mem_len, old.shape[1] + cur.shape[1])
        out.append(np.stack(rows) if rows else np.zeros((0, keep) + cur.shape[2:]))
    return out


def update_rows(mem_rows: Sequence[np.ndarray], h: np.ndarray, mem_len: int
                ) -> List[np.ndarray]:
    """Per-row form of the update for rows whose memories differ in length
    (rows that reset at a document boundary, [P1] section "Batched Streams"):
    row b's memory [m_b, d] becomes Tail_mem_len([mem_b; h_b])."""
    return [tail_rows(m, hb, mem_len) for m, hb in zip(mem_rows, h)]
