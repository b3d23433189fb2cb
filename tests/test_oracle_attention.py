"""Pins of the fp64 attention oracle against what the pages fix.

Each test checks the oracle against something other than itself: a printed
example, the pages' own shift procedure, a library routine (torch's fp64
scaled_dot_product_attention) or a pure-Python brute force.
"""
import math
import os

import numpy as np
import pytest
import torch

import txl_synth
from oracle import attention as oa
from oracle import stack as ost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(t):
    return t.double().numpy()


def shift_by_reshape(x: np.ndarray) -> np.ndarray:
    """The alignment of zty624.github.io "Transformer-XL" notes, section
    "Relative Shift Trick", stated by where each output entry comes from.

    The page pads one zero column in front of the [q_len, k_len] logits,
    rereads that buffer as k_len + 1 rows of q_len, drops the first row and
    rereads the rest as [q_len, k_len]. In flat (row-major) indices: output
    entry (i, c) is entry f = q_len + i*k_len + c of the padded buffer, whose
    rows are k_len + 1 long; padded entry f sits in column f mod (k_len + 1)
    of row f div (k_len + 1), and column 0 is the zero pad while column
    b > 0 holds logit (row, b - 1)."""
    q_len, k_len = x.shape[-2:]
    out = np.zeros(x.shape)
    for i in range(q_len):
        for c in range(k_len):
            f = q_len + i * k_len + c
            row, col = divmod(f, k_len + 1)
            if col > 0:
                out[..., i, c] = x[..., row, col - 1]
    return out


def make_txl_mask(q_len: int, mem_len: int) -> np.ndarray:
    """The visible mask as the same page's section "Causal Mask With Memory"
    builds it, block by block: an all-visible [q_len, mem_len] memory block
    beside a lower-triangular [q_len, q_len] block for the current segment
    (True = visible)."""
    mask = np.zeros((q_len, mem_len + q_len), dtype=bool)
    for i in range(q_len):
        for c in range(mem_len):
            mask[i, c] = True
        for c in range(q_len):
            mask[i, mem_len + c] = c <= i
    return mask


def read_golden_mask(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cells = [c for c in line.replace("|", " ").split()]
            rows.append([c in ("m", "x") for c in cells])
    return np.array(rows, dtype=bool)


def read_golden_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = int(v)
    return out


def c1_inputs():
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32"]
    x = txl_synth.attn_inputs(cfg)
    r = ost.rel_pos_table(_f64(x["w_r"]), cfg.M, cfg.L, cfg.H, cfg.d_h)
    return cfg, x, r


# ----------------------------------------------------------------------------
# shapes and mask
# ----------------------------------------------------------------------------
def test_worked_example_score_is_4x12():
    g = read_golden_kv(os.path.join(GOLDEN, "worked_example_4x12.txt"))
    cfg, x, r = c1_inputs()
    assert (cfg.L, cfg.M) == (g["L"], g["M"])
    res = oa.rel_attn(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), r,
                      _f64(x["u"]), _f64(x["vb"]), debug=True)
    assert res["score"].shape[-2:] == (g["score_rows"], g["score_cols"])
    # memory alone holds M x d numbers
    assert x["mem"].shape[-2] * x["mem"].shape[-1] == g["cache_numbers"]
    assert x["mem"].shape[-1] == g["cache_width"]
    # query i sees all 8 memory keys plus keys 0..i
    assert res["visible"][0, 0].sum(axis=1).tolist() == [9, 10, 11, 12]


def test_mask_rule_equals_construction_equals_printed_picture():
    printed = read_golden_mask(os.path.join(GOLDEN, "mask_M3_L4.txt"))
    assert printed.shape == (4, 7)
    assert np.array_equal(oa.visible_mask(4, 3), printed)
    assert np.array_equal(make_txl_mask(4, 3), printed)
    for L, M in [(1, 0), (5, 0), (3, 7), (8, 2), (16, 16)]:
        assert np.array_equal(oa.visible_mask(L, M), make_txl_mask(L, M))


def test_mask_partial_memory():
    # valid < M hides the oldest M - valid memory keys, nothing else
    L, M = 5, 6
    for valid in range(M + 1):
        m = oa.visible_mask(L, M, valid)
        full = make_txl_mask(L, M)
        assert not m[:, : M - valid].any()
        assert np.array_equal(m[:, M - valid:], full[:, M - valid:])


# ----------------------------------------------------------------------------
# relative distance indexing
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,M", [(4, 8), (4, 3), (1, 0), (6, 0), (5, 11), (9, 9)])
def test_shift_procedure_aligns_distance_labels(L, M):
    """Golden test of the shift ([P1] "Relative Shift Golden Test"): label
    R row t with its distance M+L-1-t, shift the raw logits with the page's
    procedure, and every visible entry must carry the distance i - j."""
    labels = (M + L - 1) - np.arange(M + L, dtype=np.float64)
    raw = np.broadcast_to(labels, (L, M + L)).copy()
    shifted = shift_by_reshape(raw)
    vis = make_txl_mask(L, M)
    assert np.array_equal(shifted[vis], oa.rel_ids(L, M)[vis].astype(float))


@pytest.mark.parametrize("L,M,valid", [(4, 8, 8), (7, 5, 3), (3, 0, 0), (6, 6, 0)])
def test_oracle_position_term_reads_distance(L, M, valid):
    """With q = e0, k = u = v = 0 and R[t] = (M+L-1-t) e0, the oracle's
    content-position term must equal the closed-form distance i - j."""
    dh = 4
    q = np.zeros((1, 1, L, dh)); q[..., 0] = 1.0
    k = np.zeros((1, 1, M + L, dh))
    v = np.random.default_rng(0).standard_normal((1, 1, M + L, dh))
    r = np.zeros((1, M + L, dh)); r[0, :, 0] = (M + L - 1) - np.arange(M + L)
    z = np.zeros((1, dh))
    res = oa.rel_attn(q, k, v, r, z, z, valid=[valid], debug=True)
    vis = res["visible"][0, 0]
    assert np.array_equal(vis, oa.visible_mask(L, M, valid))
    assert np.array_equal(res["cp"][0, 0][vis], oa.rel_ids(L, M)[vis].astype(float))


def test_position_term_is_toeplitz():
    """Translation invariance ([P1] "Dimension Walkthrough", shifting query
    and key by the same offset keeps i - j): the position terms of (i, j)
    and (i+1, j+1) are equal whenever both are visible."""
    cfg, x, r = c1_inputs()
    res = oa.rel_attn(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), r,
                      _f64(x["u"]), _f64(x["vb"]), debug=True)
    gp = res["gp"][0, 0]
    vis = res["visible"][0, 0]
    L, ML = gp.shape
    n = 0
    for i in range(L - 1):
        for jp in range(ML - 1):
            if vis[i, jp] and vis[i + 1, jp + 1]:
                assert abs(gp[i, jp] - gp[i + 1, jp + 1]) <= 1e-14 * abs(gp[i, jp])
                n += 1
    assert n > 0


# ----------------------------------------------------------------------------
# the four-term score
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,M,valid", [(4, 8, 8), (6, 5, 2), (5, 0, 0)])
def test_four_terms_equal_factored_form_through_shift(L, M, valid):
    """The oracle sums the four terms of [P1] "Relative Positional Encoding"
    separately, looking R up by distance. The factored (q+u).k + (q+v).R form
    of [P3] section 2.2, with the position part aligned by the page's shift
    procedure instead of a lookup, must give the same score."""
    rng = np.random.default_rng(L * 100 + M)
    dh = 8
    q = rng.standard_normal((1, 1, L, dh))
    k = rng.standard_normal((1, 1, M + L, dh))
    v = rng.standard_normal((1, 1, M + L, dh))
    r = rng.standard_normal((1, M + L, dh))
    u = rng.standard_normal((1, dh))
    vb = rng.standard_normal((1, dh))
    res = oa.rel_attn(q, k, v, r, u, vb, valid=[valid], debug=True)
    content = (q[0, 0] + u[0]) @ k[0, 0].T
    position = shift_by_reshape((q[0, 0] + vb[0]) @ r[0].T)
    vis = oa.visible_mask(L, M, valid)
    np.testing.assert_allclose(res["score"][0, 0][vis], (content + position)[vis],
                               rtol=1e-12, atol=1e-12)
    assert np.isnan(res["score"][0, 0][~vis]).all()


# ----------------------------------------------------------------------------
# reductions to standard attention (torch fp64 SDPA on the CPU)
# ----------------------------------------------------------------------------
def _sdpa(q, k, v, mask, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(mask), scale=scale).numpy()


def test_no_memory_is_causal_attention_with_relative_bias():
    """M = 0: causal softmax attention whose additive bias is
    u.k_j + (q_i+v).R_{i-j}, the bias aligned with the page's shift."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M0"]
    x = txl_synth.attn_inputs(cfg, B=2, H=3, L=37)
    L, dh = 37, cfg.d_h
    r = ost.rel_pos_table(_f64(x["w_r"])[:, : 3 * dh], 0, L, 3, dh)
    q, k, v = _f64(x["q"]), _f64(x["k"]), _f64(x["v"])
    u, vb = _f64(x["u"]), _f64(x["vb"])
    scale = 1.0 / math.sqrt(dh)
    res = oa.rel_attn(q, k, v, r, u, vb, valid=[0, 0])
    bias = np.empty((2, 3, L, L))
    for b in range(2):
        for h in range(3):
            bias[b, h] = (k[b, h] @ u[h])[None, :] + shift_by_reshape(
                (q[b, h] + vb[h]) @ r[h].T)
    causal = np.tril(np.ones((L, L), dtype=bool))
    mask = np.where(causal, bias * scale, -np.inf)
    ref = _sdpa(q, k, v, mask, scale)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("valid_mode", ["full", "mixed"])
def test_zero_bias_zero_r_is_standard_masked_attention(valid_mode):
    """u = v = 0 and R = 0: standard softmax attention under the rectangular
    visible mask (memory block beside the causal block)."""
    B, H, L, M, dh = 3, 2, 11, 7, 16
    rng = np.random.default_rng(3)
    q = rng.standard_normal((B, H, L, dh))
    k = rng.standard_normal((B, H, M + L, dh))
    v = rng.standard_normal((B, H, M + L, dh))
    z = np.zeros((H, dh))
    r = np.zeros((H, M + L, dh))
    valid = txl_synth.valid_counts(B, M, valid_mode).numpy()
    res = oa.rel_attn(q, k, v, r, z, z, valid=valid)
    mask = np.zeros((B, 1, L, M + L), dtype=bool)
    for b in range(B):
        m = make_txl_mask(L, M)
        m[:, : M - valid[b]] = False
        mask[b, 0] = m
    ref = _sdpa(q, k, v, mask, 1.0 / math.sqrt(dh))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# brute force and invariants
# ----------------------------------------------------------------------------
def _brute(q, k, v, r, u, vb, M, valid, scale):
    """Pure-Python enumeration for one (batch, head) on tiny inputs."""
    L, dh = len(q), len(q[0])
    dot = lambda a, b: sum(a[e] * b[e] for e in range(dh))
    out = []
    for i in range(L):
        s = {}
        for jp in range(M + L):
            j = jp - M
            if (j < 0 and j >= -valid) or (0 <= j <= i):
                rr = r[(M + L - 1) - (i - j)]
                s[jp] = (dot(q[i], k[jp]) + dot(q[i], rr) + dot(u, k[jp])
                         + dot(vb, rr)) * scale
        mx = max(s.values())
        w = {jp: math.exp(val - mx) for jp, val in s.items()}
        z = sum(w.values())
        out.append([sum(w[jp] / z * v[jp][e] for jp in w) for e in range(dh)])
    return out


@pytest.mark.parametrize("L", [1, 2, 3])
@pytest.mark.parametrize("M", [0, 1, 3])
@pytest.mark.parametrize("dh", [1, 4])
def test_brute_force_tiny(L, M, dh):
    rng = np.random.default_rng(L * 31 + M * 7 + dh)
    q = rng.standard_normal((1, 1, L, dh))
    k = rng.standard_normal((1, 1, M + L, dh))
    v = rng.standard_normal((1, 1, M + L, dh))
    r = rng.standard_normal((1, M + L, dh))
    u = rng.standard_normal((1, dh))
    vb = rng.standard_normal((1, dh))
    for valid in range(M + 1):
        res = oa.rel_attn(q, k, v, r, u, vb, valid=[valid], scale=0.7)
        ref = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                     r[0].tolist(), u[0].tolist(), vb[0].tolist(), M, valid, 0.7)
        np.testing.assert_allclose(res["out"][0, 0], np.array(ref),
                                   rtol=1e-12, atol=1e-13)


def test_softmax_rows_sum_to_one_and_masked_weights_are_zero():
    cfg, x, r = c1_inputs()
    for valid in (8, 5, 0):
        res = oa.rel_attn(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), r,
                          _f64(x["u"]), _f64(x["vb"]), valid=[valid], debug=True)
        p, vis = res["p"][0, 0], res["visible"][0, 0]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (p[~vis] == 0.0).all()
        assert (p[vis] > 0.0).all()
        # lse is the log normaliser of the scaled visible scores
        s = res["score"][0, 0] / math.sqrt(cfg.d_h)
        for i in range(cfg.L):
            ref = math.log(np.exp(s[i][vis[i]]).sum())
            assert abs(res["lse"][0, 0, i] - ref) < 1e-12


def test_rows_and_heads_are_independent():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = txl_synth.attn_inputs(cfg, B=3, H=2, L=9, M=6)
    q, k, v = _f64(x["q"]), _f64(x["k"]), _f64(x["v"])
    u, vb = _f64(x["u"]), _f64(x["vb"])
    r = np.random.default_rng(1).standard_normal((2, 15, cfg.d_h))
    valid = np.array([6, 2, 0])
    base = oa.rel_attn(q, k, v, r, u, vb, valid=valid)["out"]
    pb = [2, 0, 1]
    perm = oa.rel_attn(q[pb], k[pb], v[pb], r, u, vb, valid=valid[pb])["out"]
    assert np.array_equal(perm, base[pb])
    ph = [1, 0]
    perm_h = oa.rel_attn(q[:, ph], k[:, ph], v[:, ph], r[ph], u[ph], vb[ph],
                         valid=valid)["out"]
    assert np.array_equal(perm_h, base[:, ph])


def test_attn_flops_counts_visible_pairs():
    # L=4, M=8 full memory: 4*8 memory pairs + 10 causal pairs = 42
    assert oa.attn_flops(1, 1, 4, 64, [8]) == 6 * 64 * 42
    vis = oa.visible_mask(4, 8, 5)
    assert oa.attn_flops(1, 1, 4, 64, [5]) == 6 * 64 * vis.sum()
