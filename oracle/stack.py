"""fp64 oracle: the relative-position table, one layer, one segment, a stream.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

What the pages fix, and what is a stated reading:
  * Q from the current segment only, K and V from [SG(mem); H] ([P1]
    "Transformer-XL" notes, sections "Segment-Level Recurrence" and "Batched
    Tensor Contract"; [P2] "019 Transformer-XL", section 3 pseudo-code).
  * Layer n reads the memory of layer n-1 and every layer keeps its own
    memory list [M^(0) ... M^(N)] updated with Tail_M ([P1] "Segment-Level
    Recurrence"; [P2] section 2 on the dependency moving down one layer per
    segment).
  * Rows reset at document boundaries start from an empty memory ([P1]
    "Training Loop Sketch" sets mems to None on reset; "Batched Streams" makes
    the flag per row).
  * R is a sinusoidal embedding of the relative distance projected per head
    ([P4] "Transformer-XL" glossary entries on the four-term score). The
    sinusoid's formula is not printed: the reading used here (and stated as
    parity unpinned) is the concatenated [sin | cos] form with frequencies
    10000^(-2k/d), k = 0 .. d/2-1.
  * The rest of the layer is not on the pages. Reading used (parity
    unpinned): attention output projection W^O, residual, LayerNorm (biased
    variance, eps 1e-5); feed-forward d -> d_ff -> d with the exact erf GELU,
    residual, LayerNorm. No biases, no dropout, no absolute positions.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf

from .attention import rel_attn, rel_attn_bwd
from .memory import tail_rows

LN_EPS = 1e-5


def sinusoid(dist: np.ndarray, d: int) -> np.ndarray:
    """Sinusoidal embedding [len(dist), d] of the distances ``dist``.

    emb(delta) = [sin(delta * f_0..f_{d/2-1}) | cos(delta * f_0..f_{d/2-1})],
    f_k = 10000^(-2k/d). (Reading; the pages only say "sinusoidal".)
    """
    assert d % 2 == 0
    dist = np.asarray(dist, dtype=np.float64)
    k = np.arange(d // 2, dtype=np.float64)
    freq = 10000.0 ** (-2.0 * k / d)
    ang = dist[:, None] * freq[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def rel_pos_table(w_r: np.ndarray, M: int, L: int, H: int, dh: int
                  ) -> np.ndarray:
    """R for every head: [H, M+L, dh] with row t holding distance M+L-1-t.

    [P1] "Dimension Walkthrough": R has one row per relative distance, from
    the farthest memory slot to the current position. Each head projects the
    sinusoid with its own slice of W_R [d, H*dh] (math orientation).
    """
    w_r = np.asarray(w_r, dtype=np.float64)
    d = w_r.shape[0]
    dist = np.arange(M + L - 1, -1, -1)
    s = sinusoid(dist, d)
    r = s @ w_r
    return r.reshape(M + L, H, dh).transpose(1, 0, 2).copy()


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray,
               eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: biased variance, then gain and shift."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) with the Gaussian CDF written through erf."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def _f64(w: Dict[str, object]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}


def split_heads(x: np.ndarray, H: int, dh: int) -> np.ndarray:
    """[n, H*dh] -> [H, n, dh]: head h owns columns h*dh .. (h+1)*dh - 1
    ([P1] "Dimension Walkthrough": the projections are cut into H heads of
    d_h)."""
    n = x.shape[0]
    out = np.empty((H, n, dh))
    for h in range(H):
        out[h] = x[:, h * dh:(h + 1) * dh]
    return out


def merge_heads(x: np.ndarray) -> np.ndarray:
    """[H, n, dh] -> [n, H*dh], the inverse of split_heads."""
    H, n, dh = x.shape
    out = np.empty((n, H * dh))
    for h in range(H):
        out[:, h * dh:(h + 1) * dh] = x[h]
    return out


def r_for_memory(r_table: np.ndarray, M: int, m: int) -> np.ndarray:
    """The rows of a capacity-M table ([H, M+L, dh], row t = distance
    M+L-1-t) that a memory of m <= M stored states needs: distances m+L-1 ..
    0, i.e. rows M-m .. M+L-1 ([P1] "Dimension Walkthrough": R covers the
    distances from the farthest key present to the current position)."""
    r_table = np.asarray(r_table, dtype=np.float64)
    return r_table[:, M - m:, :]


def context(mem: np.ndarray, h: np.ndarray) -> np.ndarray:
    """The extended context [SG(mem); h] the keys and values are projected
    from: the stored memory first (oldest first), then the current segment
    ([P1] "Segment-Level Recurrence", "Batched Tensor Contract")."""
    return np.concatenate([mem, h], axis=0)


def add_norm(x: np.ndarray, f: np.ndarray, g: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Residual then LayerNorm (post-LN): LN(x + f)."""
    return layer_norm(x + f, g, b)


def layer_forward(h: np.ndarray, mem: np.ndarray, lw: Dict[str, np.ndarray],
                  r_table: np.ndarray, M: int, H: int, dh: int) -> np.ndarray:
    """One layer for one batch row.

    h [L, d] is H^(n-1) of the current segment, mem [m, d] (m <= M) the
    memory of layer n-1, oldest first. r_table is the layer's R for a memory
    of capacity M ([H, M+L, dh]); with m < M stored states only its last m+L
    rows (distances m+L-1 .. 0) are used.
    Weights in math orientation: y = x W with W [in, out].
    Steps: Q from h, K and V from [SG(mem); h] ([P1] "Segment-Level
    Recurrence"; [P2] section 3), the relative attention of each head, then
    (reading) X = LN1(h + A W^O), out = LN2(X + GELU(X W1) W2).
    """
    lw = _f64(lw)
    h = np.asarray(h, dtype=np.float64)
    mem = np.asarray(mem, dtype=np.float64)
    m = mem.shape[0]
    ext = context(mem, h)                            # [SG(mem); H]
    q = split_heads(h @ lw["wq"], H, dh)[None]
    k = split_heads(ext @ lw["wk"], H, dh)[None]
    v = split_heads(ext @ lw["wv"], H, dh)[None]
    r = r_for_memory(r_table, M, m)
    att = rel_attn(q, k, v, r, lw["u"], lw["vb"], valid=[m])["out"][0]
    a = merge_heads(att) @ lw["wo"]
    h1 = add_norm(h, a, lw["ln1_g"], lw["ln1_b"])
    f = gelu(h1 @ lw["w1"]) @ lw["w2"]
    return add_norm(h1, f, lw["ln2_g"], lw["ln2_b"])


def segment_step_row(tokens: np.ndarray, mems: Sequence[np.ndarray],
                     emb: np.ndarray, layers: Sequence[Dict[str, np.ndarray]],
                     r_tables: Sequence[np.ndarray], M: int, H: int, dh: int):
    """One segment of one batch row through the stack.

    mems is the list [M^(0) ... M^(N)] of that row (arrays [m_n, d]).
    Returns (hs, new_mems): hs = [H^(0) ... H^(N)] ([L, d] each, H^(0) the
    embedded tokens) and new_mems[n] = Tail_M([M^(n); H^(n)]).
    """
    emb = np.asarray(emb, dtype=np.float64)
    h = emb[np.asarray(tokens, dtype=np.int64)]
    hs = [h]
    for n, lw in enumerate(layers):
        h = layer_forward(h, mems[n], lw, r_tables[n], M, H, dh)
        hs.append(h)
    new_mems = [tail_rows(mems[n], hs[n], M) for n in range(len(layers) + 1)]
    return hs, new_mems


def stream(tokens: np.ndarray, resets: np.ndarray, emb: np.ndarray,
           layers: Sequence[Dict[str, np.ndarray]],
           r_tables: Sequence[np.ndarray], M: int, H: int, dh: int,
           rows: Optional[Sequence[int]] = None) -> List[Dict[int, List[np.ndarray]]]:
    """Stream consecutive segments through the stack, row by row.

    tokens [S, B, L] ints; resets [S, B] flags. A row whose flag is set (and
    every row at its first segment) starts from empty memories, as with
    mems = None in [P1] "Training Loop Sketch". Returns, per segment, a dict
    row -> [H^(0) ... H^(N)].
    """
    tokens = np.asarray(tokens)
    resets = np.asarray(resets)
    S, B, _ = tokens.shape
    rows = list(range(B)) if rows is None else list(rows)
    d = np.asarray(emb).shape[1]
    n_mem = len(layers) + 1
    mems: Dict[int, Optional[List[np.ndarray]]] = {b: None for b in rows}
    out = []
    for s in range(S):
        seg = {}
        for b in rows:
            if mems[b] is None or resets[s, b]:
                mems[b] = [np.zeros((0, d)) for _ in range(n_mem)]
            hs, mems[b] = segment_step_row(tokens[s, b], mems[b], emb, layers,
                                           r_tables, M, H, dh)
            seg[b] = hs
        out.append(seg)
    return out


# ----------------------------------------------------------------------------
# gradients of one segment (training)
# ----------------------------------------------------------------------------
def gelu_grad(x: np.ndarray) -> np.ndarray:
    """d/dx of the exact GELU x Phi(x): Phi(x) + x phi(x)."""
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def layer_norm_backward(x: np.ndarray, g: np.ndarray, dy: np.ndarray, eps: float = LN_EPS):
    """Gradients of y = layer_norm(x, g, b) over the last axis: returns
    (dx, dg, db) for the incoming dy, written out by the chain rule through
    the mean and the biased variance (xhat = (x - mean) r, r = 1/sqrt(var+eps)):
        dg = sum_rows dy xhat,   db = sum_rows dy,
        dx = r (gdy - mean(gdy) - xhat mean(gdy xhat)),  gdy = dy g."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xhat = (x - mu) * r
    gdy = dy * g
    dx = r * (gdy - gdy.mean(axis=-1, keepdims=True)
              - xhat * (gdy * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def layer_backward(h: np.ndarray, mem: np.ndarray, lw: Dict[str, np.ndarray],
                   wr: np.ndarray, M: int, H: int, dh: int, dy: np.ndarray):
    """Gradients of one layer (layer_forward) for one batch row.

    dy [L, d] is the gradient arriving at the layer's output. The memory is
    a stop-gradient input ([P1] "Why Stop Gradient"; [P2] section
    "stop-gradient到底切断哪里"): nothing is returned for it, but the keys and
    values projected from its rows are part of this segment's computation,
    so W^K and W^V receive their gradient from the memory rows as well.
    R is built from the layer's W_R (wr [d, H*dh], math orientation) as in
    rel_pos_table, so W_R gets its gradient through R.

    Returns (dh_in [L, d], grads) with grads holding one array per weight of
    layer_forward (wq, wk, wv, wo, wr, u, vb, ln1_g, ln1_b, w1, w2, ln2_g,
    ln2_b), each the exact derivative of sum(dy * out) in float64.
    """
    lw = _f64(lw)
    h = np.asarray(h, dtype=np.float64)
    mem = np.asarray(mem, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    L, d = h.shape
    m = mem.shape[0]
    # forward, keeping what the backward needs
    r_table = rel_pos_table(wr, M, L, H, dh)
    ext = context(mem, h)
    q = split_heads(h @ lw["wq"], H, dh)[None]
    k = split_heads(ext @ lw["wk"], H, dh)[None]
    v = split_heads(ext @ lw["wv"], H, dh)[None]
    r = r_for_memory(r_table, M, m)
    att = rel_attn(q, k, v, r, lw["u"], lw["vb"], valid=[m])["out"][0]
    o = merge_heads(att)
    x1 = h + o @ lw["wo"]
    h1 = layer_norm(x1, lw["ln1_g"], lw["ln1_b"])
    fpre = h1 @ lw["w1"]
    f = gelu(fpre)
    x2 = h1 + f @ lw["w2"]
    # backward
    g = {}
    dx2, g["ln2_g"], g["ln2_b"] = layer_norm_backward(x2, lw["ln2_g"], dy)
    g["w2"] = f.T @ dx2
    dfpre = (dx2 @ lw["w2"].T) * gelu_grad(fpre)
    g["w1"] = h1.T @ dfpre
    dh1 = dfpre @ lw["w1"].T + dx2
    dx1, g["ln1_g"], g["ln1_b"] = layer_norm_backward(x1, lw["ln1_g"], dh1)
    g["wo"] = o.T @ dx1
    datt = split_heads(dx1 @ lw["wo"].T, H, dh)[None]
    ag = rel_attn_bwd(q, k, v, r, lw["u"], lw["vb"], datt, valid=[m])
    dq = merge_heads(ag["dq"][0])
    dk = merge_heads(ag["dk"][0])
    dv = merge_heads(ag["dv"][0])
    g["wq"] = h.T @ dq
    g["wk"] = ext.T @ dk          # memory rows included: they feed W^K ...
    g["wv"] = ext.T @ dv
    g["u"] = ag["du"]
    g["vb"] = ag["dvb"]
    # ... but the gradient stops there: only the segment rows reach h
    dh_in = dq @ lw["wq"].T + dk[m:] @ lw["wk"].T + dv[m:] @ lw["wv"].T + dx1
    # W_R: R[h] = S W_R[:, head h] with S the sinusoid of distances M+L-1..0;
    # the table rows a memory of m states uses are its last m+L
    dr_full = np.zeros_like(r_table)
    dr_full[:, M - m:, :] = ag["dr"]
    s = sinusoid(np.arange(M + L - 1, -1, -1), d)
    g["wr"] = s.T @ merge_heads(dr_full)
    return dh_in, g


def segment_backward_row(tokens: np.ndarray, mems: Sequence[np.ndarray], emb: np.ndarray,
                         layers: Sequence[Dict[str, np.ndarray]], M: int, H: int, dh: int,
                         dy: np.ndarray):
    """Gradients of one segment of one batch row through the stack for the
    gradient dy [L, d] arriving at H^(N): runs the forward (segment_step_row,
    R built from each layer's W_R), then the layers in reverse, and
    scatters the gradient reaching H^(0) into the embedding rows of the
    tokens (a token that occurs twice adds twice). The memories are
    stop-gradient inputs. Returns (demb [vocab, d], [grads of layer 1 .. N])."""
    emb = np.asarray(emb, dtype=np.float64)
    L = len(tokens)
    r_tables = [rel_pos_table(lw["wr"], M, L, H, dh) for lw in layers]
    hs, _ = segment_step_row(tokens, mems, emb, layers, r_tables, M, H, dh)
    grads = [None] * len(layers)
    g_h = np.asarray(dy, dtype=np.float64)
    for n in range(len(layers) - 1, -1, -1):
        g_h, grads[n] = layer_backward(hs[n], mems[n], layers[n], layers[n]["wr"], M, H, dh, g_h)
    demb = np.zeros_like(emb)
    for pos, t in enumerate(np.asarray(tokens, dtype=np.int64)):
        demb[t] += g_h[pos]
    return demb, grads
