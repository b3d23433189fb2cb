"""fp64 oracle: relative-position attention over [memory; current segment].

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

Conventions, read from [P1] "Transformer-XL" notes:
  * Key positions run from -M (oldest memory slot) to L-1 (last token of the
    current segment); query positions run from 0 to L-1
    (section "Causal Mask With Memory", the key-position listing).
  * Arrays hold keys in that logical order: index j' = j + M.
  * R holds one row per relative distance, from the farthest memory slot down
    to distance 0 (section "Dimension Walkthrough": R covers the distances
    from the farthest memory to the current segment). Row t therefore holds
    distance M+L-1-t; this module looks the row up by distance and never uses
    the pad/reshape/slice shift.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def allow(i, j, valid):
    """Visibility of key position j for query position i.

    [P1] section "Causal Mask With Memory", rule allow(i, j): memory keys
    (j < 0) are visible, current keys are visible for 0 <= j <= i and masked
    for j > i. A row's memory holds only ``valid`` states: slots farther back
    than that (a stream that has not filled its memory yet, or a row that
    just started a new document, which [P1] says must be cleared or masked)
    are masked too, so memory is visible for -valid <= j < 0.
    Works elementwise on numpy arrays.
    """
    j = np.asarray(j)
    mem_visible = (j < 0) & (j >= -valid)
    cur_visible = (j >= 0) & (j <= i)
    return mem_visible | cur_visible


def visible_mask(L: int, M: int, valid: Optional[int] = None) -> np.ndarray:
    """The [L, M+L] boolean visibility matrix (True = visible)."""
    valid = M if valid is None else valid
    j = np.arange(-M, L)
    return np.stack([allow(i, j, valid) for i in range(L)], axis=0)


def rel_ids(L: int, M: int) -> np.ndarray:
    """Relative distance i - j for every (query i, key position j).

    [P1] section "Relative Shift Golden Test": queries sit at positions
    0..L-1 and keys at -M..L-1, and the target of entry (i, j) is the
    distance i - j. Written out per entry: logical key index j' holds key
    position j = j' - M.
    """
    ids = np.zeros((L, M + L), dtype=np.int64)
    for i in range(L):
        for jp in range(M + L):
            j = jp - M
            ids[i, jp] = i - j
    return ids


def rel_attn(q, k, v, r, u, vb, valid=None, scale: Optional[float] = None,
             debug: bool = False) -> Dict[str, np.ndarray]:
    """Relative-position attention of the current segment over [mem; H].

    Shapes (float64): q [B,H,L,dh]; k, v [B,H,M+L,dh] in logical key order;
    r [H,M+L,dh] (row t = distance M+L-1-t); u, vb [H,dh]; valid [B] ints in
    [0, M] (None = all M valid); scale defaults to 1/sqrt(dh).

    For each query i and each visible key position j ([P1] "Causal Mask With
    Memory"), the score is the sum of the four terms of [P1] section
    "Relative Positional Encoding":
        content-content   q_i . k_j
        content-position  q_i . R_{i-j}
        global content    u . k_j
        global position   v . R_{i-j}
    where u and v are the per-head biases. The probabilities are the softmax
    of score*scale over visible keys only, and the output is their weighted
    sum of v_j ([P1] "Dimension Walkthrough": softmax((A + M_causal)/sqrt(dh)) V,
    with the additive mask -inf on hidden keys, so hidden keys get weight 0).

    Returns {"out" [B,H,L,dh], "lse" [B,H,L]} (lse = natural-log
    log-sum-exp of the scaled visible scores); with ``debug`` also the raw
    score A [B,H,L,M+L] (NaN where hidden), its four terms, the
    probabilities (0 where hidden) and the visibility mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    vb = np.asarray(vb, dtype=np.float64)
    B, H, L, dh = q.shape
    M = k.shape[2] - L
    assert M >= 0 and k.shape == (B, H, M + L, dh) and v.shape == k.shape
    assert r.shape == (H, M + L, dh) and u.shape == (H, dh) and vb.shape == (H, dh)
    if valid is None:
        valid = np.full((B,), M, dtype=np.int64)
    valid = np.asarray(valid, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(dh)

    out = np.zeros((B, H, L, dh))
    lse = np.zeros((B, H, L))
    if debug:
        shp = (B, H, L, M + L)
        dbg = {name: np.full(shp, np.nan) for name in
               ("score", "cc", "cp", "gc", "gp")}
        dbg["p"] = np.zeros(shp)
        dbg["visible"] = np.zeros(shp, dtype=bool)

    key_pos = np.arange(-M, L)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                vis = allow(i, key_pos, int(valid[b]))
                jp = np.nonzero(vis)[0]          # logical key indices
                j = jp - M                       # key positions
                dist = i - j                     # relative distance i - j
                r_d = r[h, (M + L - 1) - dist]   # R_{i-j}, looked up by distance
                qi = q[b, h, i]
                kj = k[b, h, jp]
                cc = kj @ qi
                cp = r_d @ qi
                gc = kj @ u[h]
                gp = r_d @ vb[h]
                a = cc + cp + gc + gp
                s = a * scale
                smax = s.max()
                e = np.exp(s - smax)
                z = e.sum()
                p = e / z
                out[b, h, i] = p @ v[b, h, jp]
                lse[b, h, i] = smax + math.log(z)
                if debug:
                    dbg["score"][b, h, i, jp] = a
                    dbg["cc"][b, h, i, jp] = cc
                    dbg["cp"][b, h, i, jp] = cp
                    dbg["gc"][b, h, i, jp] = gc
                    dbg["gp"][b, h, i, jp] = gp
                    dbg["p"][b, h, i, jp] = p
                    dbg["visible"][b, h, i] = vis
    res = {"out": out, "lse": lse}
    if debug:
        res.update(dbg)
    return res


def attn_flops(B: int, H: int, L: int, dh: int, valid) -> float:
    """Algorithmic flops of one call: three contractions (q.k, q.R, p.v) of
    2*dh flops each per visible (query, key) pair; masked pairs are not work.
    Visible pairs of row b: L*valid_b (memory) + L(L+1)/2 (causal segment).
    """
    valid = np.asarray(valid, dtype=np.int64).reshape(-1)
    if valid.size == 1 and B > 1:
        valid = np.full((B,), int(valid[0]))
    pairs = float(np.sum(L * valid + L * (L + 1) // 2))
    return 6.0 * dh * H * pairs


def rel_attn_bwd(q, k, v, r, u, vb, dout, valid=None,
                 scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Exact gradients of ``rel_attn``'s output with respect to every input.

    ``dout`` [B,H,L,dh] is the gradient arriving at ``out``; the result holds
    dq [B,H,L,dh], dk and dv [B,H,M+L,dh], dr [H,M+L,dh], du and dvb [H,dh].

    The forward is the one of ``rel_attn`` (four-term score of [P1]
    "Relative Positional Encoding" regrouped as (q+u).k + (q+v).R_{i-j}
    ([P3] section 2.2), softmax over the keys allowed by [P1] "Causal Mask
    With Memory"); this is its derivative written out per query with the
    chain rule, in float64:
        dp_j  = dout_i . v_j
        ds_j  = p_j (dp_j - sum_k p_k dp_k)        (softmax Jacobian)
        g_j   = ds_j * scale                       (gradient of the raw score)
        dq_i += sum_j g_j (k_j + R_{i-j})
        dk_j += g_j (q_i + u),   dv_j += p_j dout_i
        dR_{i-j} += g_j (q_i + v)                  (row looked up by distance)
        du   += sum_j g_j k_j,   dvb += sum_j g_j R_{i-j}
    Memory keys get dk / dv like any other key: the stop-gradient of [P1]
    "Why Stop Gradient" and [P2] section "stop-gradient到底切断哪里" cuts the
    path back into the earlier segment that produced the memory, not the
    gradient of this segment's keys and values (which still reaches W_K and
    W_V). Hidden keys get exactly zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    vb = np.asarray(vb, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, L, dh = q.shape
    M = k.shape[2] - L
    assert M >= 0 and k.shape == (B, H, M + L, dh) and v.shape == k.shape
    assert r.shape == (H, M + L, dh) and dout.shape == q.shape
    if valid is None:
        valid = np.full((B,), M, dtype=np.int64)
    valid = np.asarray(valid, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(dh)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dr = np.zeros_like(r)
    du = np.zeros_like(u)
    dvb = np.zeros_like(vb)
    key_pos = np.arange(-M, L)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                jp = np.nonzero(allow(i, key_pos, int(valid[b])))[0]
                rows = (M + L - 1) - (i - (jp - M))      # R row of each key's distance
                r_d = r[h, rows]
                kj = k[b, h, jp]
                s = (kj @ (q[b, h, i] + u[h]) + r_d @ (q[b, h, i] + vb[h])) * scale
                e = np.exp(s - s.max())
                p = e / e.sum()
                dp = v[b, h, jp] @ dout[b, h, i]
                ds = p * (dp - p @ dp)
                g = ds * scale
                dq[b, h, i] += g @ kj + g @ r_d
                dk[b, h, jp] += np.outer(g, q[b, h, i] + u[h])
                dv[b, h, jp] += np.outer(p, dout[b, h, i])
                dr[h, rows] += np.outer(g, q[b, h, i] + vb[h])   # rows distinct per query
                du[h] += g @ kj
                dvb[h] += g @ r_d
    return {"dq": dq, "dk": dk, "dv": dv, "dr": dr, "du": du, "dvb": dvb}


def attn_bwd_flops(B: int, H: int, L: int, dh: int, valid) -> float:
    """Algorithmic flops of the backward: the two score contractions
    recomputed (q.k, q.R) and the six gradient contractions (dout.v, p.dout,
    g.k, g.R, g.(q+u), g.(q+v)), 2*dh flops each per visible pair."""
    return attn_flops(B, H, L, dh, valid) * 8.0 / 3.0
