"""Pins of the fp64 attention-backward oracle.

``oracle.attention.rel_attn_bwd`` writes the chain rule out by hand; these
tests check it against things that do not share that derivation:
  * central finite differences of the (separately pinned) forward oracle,
    element by element for every input, on tiny shapes;
  * torch fp64 autograd of an independent dense formulation (full score
    matrix, relative term gathered by distance, additive -inf mask);
  * identities the mathematics fixes: every row of probabilities sums to 1
    (so sum_j dv_j = sum_i dout_i, and the score gradients of a row sum to 0,
    so sum_j dk_j = 0 and sum_t dR_t = 0), du + dvb = sum_i dq_i, hidden keys
    get zero gradient, and a row reset to no memory gives the gradients of a
    run without memory.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa

NAMES = ("q", "k", "v", "r", "u", "vb")


def draw(B, H, L, M, dh, seed, valid=None):
    g = np.random.default_rng(seed)
    x = {
        "q": g.normal(size=(B, H, L, dh)),
        "k": g.normal(size=(B, H, M + L, dh)),
        "v": g.normal(size=(B, H, M + L, dh)),
        "r": g.normal(size=(H, M + L, dh)),
        "u": g.normal(size=(H, dh)) * 0.5,
        "vb": g.normal(size=(H, dh)) * 0.5,
        "dout": g.normal(size=(B, H, L, dh)),
    }
    x["valid"] = np.full(B, M) if valid is None else np.asarray(valid)
    return x


def fwd_loss(x, scale=None):
    o = oa.rel_attn(*(x[n] for n in NAMES), valid=x["valid"], scale=scale)["out"]
    return float(np.sum(o * x["dout"]))


def grads(x, scale=None):
    return oa.rel_attn_bwd(*(x[n] for n in NAMES), x["dout"], valid=x["valid"], scale=scale)


@pytest.mark.parametrize("B,H,L,M,dh,valid,seed", [
    (1, 1, 3, 2, 4, None, 0),
    (2, 2, 3, 3, 3, [1, 0], 1),
    (1, 2, 4, 0, 2, None, 2),
])
def test_finite_differences(B, H, L, M, dh, valid, seed):
    x = draw(B, H, L, M, dh, seed, valid)
    g = grads(x, scale=0.7)
    eps = 1e-6
    worst = 0.0
    for name in NAMES:
        gname = "d" + name
        flat = x[name].reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + eps
            fp = fwd_loss(x, scale=0.7)
            flat[e] = keep - eps
            fm = fwd_loss(x, scale=0.7)
            flat[e] = keep
            fd = (fp - fm) / (2 * eps)
            an = g[gname].reshape(-1)[e]
            worst = max(worst, abs(fd - an))
            assert abs(fd - an) <= 1e-7 * (1 + abs(fd)), (gname, e, fd, an)
    assert worst < 1e-7


def dense_torch(x, scale):
    """Independent formulation: the whole [L, M+L] score matrix at once, the
    position term (q+v) R^T gathered by distance, an additive -inf mask."""
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    B, H, L, dh = x["q"].shape
    ML = x["k"].shape[2]
    M = ML - L
    qu = t["q"] + t["u"][None, :, None, :]
    qv = t["q"] + t["vb"][None, :, None, :]
    content = qu @ t["k"].transpose(-1, -2)                             # [B,H,L,M+L]
    pos_all = qv @ t["r"][None].transpose(-1, -2)                       # [B,H,L,M+L] by row t
    i = torch.arange(L)[:, None]
    jp = torch.arange(ML)[None, :]
    row = (jp + L - 1 - i).clamp(0, ML - 1)                             # R row of distance i-(jp-M)
    pos = torch.gather(pos_all, 3, row.expand(B, H, L, ML))
    j = jp - M
    valid = torch.tensor(x["valid"])[:, None, None, None]
    vis = ((j < 0) & (j >= -valid)) | ((j >= 0) & (j <= i))
    s = (content + pos) * scale
    s = s.masked_fill(~vis, float("-inf"))
    out = torch.softmax(s, dim=-1) @ t["v"]
    (out * torch.tensor(x["dout"])).sum().backward()
    return {"d" + n: t[n].grad.numpy() for n in NAMES}


@pytest.mark.parametrize("B,H,L,M,valid,seed", [
    (2, 3, 16, 24, [24, 5], 3),
    (1, 2, 20, 0, None, 4),
    (3, 1, 9, 40, [0, 40, 17], 5),
])
def test_against_torch_autograd_dense(B, H, L, M, valid, seed):
    x = draw(B, H, L, M, 8, seed, valid)
    scale = 1 / math.sqrt(8)
    ref = dense_torch(x, scale)
    g = grads(x)
    for name in ref:
        err = np.abs(g[name] - ref[name]).max()
        assert err <= 1e-10 * (1 + np.abs(ref[name]).max()), (name, err)


def test_identities():
    B, H, L, M = 2, 2, 12, 10
    x = draw(B, H, L, M, 6, 6, valid=[10, 3])
    g = grads(x)
    # probabilities of a row sum to 1: sum over keys of dv = sum over queries of dout
    assert np.allclose(g["dv"].sum(axis=2), x["dout"].sum(axis=2), atol=1e-12)
    # score gradients of a row sum to 0
    assert np.abs(g["dk"].sum(axis=2)).max() < 1e-12
    assert np.abs(g["dr"].sum(axis=1)).max() < 1e-12
    # dq_i = sum_j g_j (k_j + R): summed over batch and queries it is du + dvb
    assert np.allclose(g["dq"].sum(axis=(0, 2)), g["du"] + g["dvb"], atol=1e-12)
    # hidden memory slots of row 1 (valid 3 of 10) get nothing
    assert (g["dk"][1, :, :M - 3] == 0).all() and (g["dv"][1, :, :M - 3] == 0).all()


def test_reset_row_equals_run_without_memory():
    """valid = 0 gives the gradients of the same segment with M = 0 (the
    memory rows get zero, the current rows match)."""
    B, H, L, M = 1, 2, 7, 5
    x = draw(B, H, L, M, 4, 7, valid=[0])
    g = grads(x)
    y = dict(x)
    y["k"], y["v"] = x["k"][:, :, M:], x["v"][:, :, M:]
    y["r"] = x["r"][:, M:]
    y["valid"] = np.zeros(B, dtype=np.int64)
    h = grads(y)
    assert np.abs(g["dq"] - h["dq"]).max() < 1e-13
    assert np.abs(g["dk"][:, :, M:] - h["dk"]).max() < 1e-13
    assert np.abs(g["dv"][:, :, M:] - h["dv"]).max() < 1e-13
    assert (g["dk"][:, :, :M] == 0).all()
    assert np.abs(g["dr"][:, M:] - h["dr"]).max() < 1e-13
    assert (g["dr"][:, :M] == 0).all()
    assert np.abs(g["du"] - h["du"]).max() < 1e-13 and np.abs(g["dvb"] - h["dvb"]).max() < 1e-13


def test_planted_mistakes_fail_the_pins():
    """A sign flip in the softmax Jacobian or a transposed distance lookup
    in a copy of the oracle's arithmetic is caught by the autograd pin."""
    x = draw(1, 1, 6, 4, 4, 8)
    scale = 0.5
    ref = dense_torch(x, scale)

    def broken(flip_sign, mirror_rows):
        q, k, v, r, u, vb, do = (x[n] for n in NAMES + ("dout",))
        L, M = q.shape[2], k.shape[2] - q.shape[2]
        dq = np.zeros_like(q)
        dr = np.zeros_like(r)
        for i in range(L):
            jp = np.arange(0, M + i + 1)
            rows = (M + L - 1) - (i - (jp - M))
            if mirror_rows:
                rows = (M + L - 1) - rows
            s = (k[0, 0, jp] @ (q[0, 0, i] + u[0]) + r[0, rows] @ (q[0, 0, i] + vb[0])) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            dp = v[0, 0, jp] @ do[0, 0, i]
            ds = p * (dp + p @ dp) if flip_sign else p * (dp - p @ dp)
            dq[0, 0, i] = (ds * scale) @ (k[0, 0, jp] + r[0, rows])
            dr[0, rows] += np.outer(ds * scale, q[0, 0, i] + vb[0])
        return dq, dr

    good_dq, good_dr = broken(False, False)
    assert np.abs(good_dq - ref["dq"]).max() < 1e-10
    assert np.abs(good_dr - ref["dr"]).max() < 1e-10
    for flip, mirror in ((True, False), (False, True)):
        dq, dr = broken(flip, mirror)
        assert max(np.abs(dq - ref["dq"]).max(), np.abs(dr - ref["dr"]).max()) > 1e-3
