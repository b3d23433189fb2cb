"""GPU parity of txl_rel_attn_bwd (gradients of the relative attention)
against the fp64 oracle's exact gradients on the same bf16 inputs.

Tolerance. The oracle differentiates the exact fp64 attention; the GPU
recomputes the scores from bf16 (q+u)*c and (q+v)*c (relative rounding
2^-9 each), stores p and g = scale p (dp - D) as bf16 (2^-9 each), takes
D = dout . out from the forward's bf16 output, and accumulates every
contraction in fp32. Each gradient element is a sum of such rounded
products with independent rounding errors, so its error is a few 2^-9 of
the tensor's largest element: the tests bound the normwise error
max|gpu - ref| / max|ref| by 2e-2 (about ten times 2^-9) for every output,
and require hidden memory rows to be exactly zero.
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import attention as oa
from tests.gpu_helpers import attn_case, err_report, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dr", "du", "dvb")


def gpu_grads(x, dout, kv_splits=1):
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    valid = x["valid"].to(DEV)
    B, H, L, dh = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid, lse=lse)
    grads = txl.txl_rel_attn_bwd(q, k, v, r, u, vb, out, lse, dout.to(DEV), {}, mem_valid=valid)
    torch.cuda.synchronize()
    return {n: f64(grads[n]) for n in NAMES}


def draw_dout(shape, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def oracle(x, dout, b_idx=None, h_idx=None):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    r, u, vb = f64(x["r"]), f64(x["u"]), f64(x["vb"])
    do = f64(dout)
    valid = x["valid"].numpy()
    if b_idx is not None:
        q, k, v, do, valid = q[b_idx], k[b_idx], v[b_idx], do[b_idx], valid[b_idx]
    if h_idx is not None:
        q, k, v, do = q[:, h_idx], k[:, h_idx], v[:, h_idx], do[:, h_idx]
        r, u, vb = r[h_idx], u[h_idx], vb[h_idx]
    return oa.rel_attn_bwd(q, k, v, r, u, vb, do, valid=valid)


def check(got, ref, what, names=NAMES):
    for n in names:
        assert np.isfinite(got[n]).all(), (what, n)
        rep = err_report(got[n], ref[n])
        say(f"  {what} {n}: rel_norm {rep['rel_norm']:.2e} max_abs {rep['max_abs']:.2e}")
        assert rep["rel_norm"] <= REL_TOL, (what, n, rep)


def hidden_rows_zero(got, x):
    valid = x["valid"].numpy()
    M = got["dk"].shape[2] - x["q"].shape[2]
    for b, vb in enumerate(valid):
        assert (got["dk"][b, :, :M - vb] == 0).all() and (got["dv"][b, :, :M - vb] == 0).all(), b


@pytest.mark.parametrize("valid_mode", ["full", "random"])
def test_layer_shape(valid_mode):
    """B=4 H=8 L=128 M=128 (two query tiles, four key tiles per row)."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode=valid_mode)
    dout = draw_dout(x["q"].shape, 0)
    got = gpu_grads(x, dout)
    check(got, oracle(x, dout), f"B4_H8_L128_M128 valid={valid_mode}")
    hidden_rows_zero(got, x)


@pytest.mark.parametrize("B,H,L,M,seed", [(2, 3, 100, 77, 1), (1, 2, 64, 0, 2), (3, 1, 33, 200, 3),
                                          (1, 1, 1, 0, 4), (2, 2, 130, 5, 5)])
def test_ragged_shapes(B, H, L, M, seed):
    """Partial query and key tiles, no memory, a single query, memory
    shorter than a tile; rows with random valid counts (some 0)."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, B=B, H=H, L=L, M=M, seed=seed, valid_mode="random")
    dout = draw_dout(x["q"].shape, seed)
    got = gpu_grads(x, dout)
    check(got, oracle(x, dout), f"{B}x{H} L={L} M={M}")
    hidden_rows_zero(got, x)


def test_full_size_sampled():
    """B=8 H=16 L=512 M=512 (the attention benchmark shape): rows 0 and 7 of
    heads 0 and 15 for dq, dk, dv against the oracle; dR, du, dv-bias of
    heads 0 and 15 over every row; everything finite."""
    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    x = attn_case(cfg, valid_mode="random")
    dout = draw_dout(x["q"].shape, 6)
    got = gpu_grads(x, dout)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    hidden_rows_zero(got, x)
    for h in (0, 15):
        ref = oracle(x, dout, h_idx=[h])
        sub = {n: got[n][:, [h]] for n in ("dq", "dk", "dv")}
        sub.update({n: got[n][[h]] for n in ("dr", "du", "dvb")})
        for b in (0, 7):
            check({n: sub[n][b] for n in ("dq", "dk", "dv")},
                  {n: ref[n][b] for n in ("dq", "dk", "dv")}, f"full size b={b} h={h}",
                  names=("dq", "dk", "dv"))
        check(sub, ref, f"full size h={h}", names=("dr", "du", "dvb"))


def test_identities_on_gpu():
    """Softmax identities hold for the GPU's gradients to rounding: the key
    gradients of every (b, h) sum to ~0 relative to their size, and
    sum_i dq_i over (b, i) equals du + dv-bias."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode="random", seed=9)
    dout = draw_dout(x["q"].shape, 9)
    got = gpu_grads(x, dout)
    dk_sum = np.abs(got["dk"].sum(axis=2)).max()
    assert dk_sum <= 2e-2 * np.abs(got["dk"]).max() * 8, dk_sum
    lhs = got["dq"].sum(axis=(0, 2))
    rhs = got["du"] + got["dvb"]
    assert np.abs(lhs - rhs).max() <= 1e-3 * (1 + np.abs(rhs).max())


def test_workspace_reuse_and_repeat_bitwise():
    """Two calls on one workspace (the second with fewer memory slots valid)
    give bitwise the results of fresh calls: nothing stale is read."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode="full", seed=10)
    dout = draw_dout(x["q"].shape, 10).to(DEV)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    B, H, L, dh = q.shape
    M = k.shape[2] - L
    ws = torch.empty(txl.txl_rel_attn_bwd_workspace_bytes(B, H, L, M), dtype=torch.uint8, device=DEV)

    def run(valid, workspace):
        out = torch.empty_like(q)
        lse = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid, lse=lse)
        g = txl.txl_rel_attn_bwd(q, k, v, r, u, vb, out, lse, dout, {}, mem_valid=valid,
                                 workspace=workspace)
        torch.cuda.synchronize()
        return g

    full = torch.full((B,), M, dtype=torch.int32, device=DEV)
    part = torch.tensor([M, 3, 0, 64], dtype=torch.int32, device=DEV)
    run(full, ws)
    a = run(part, ws)
    b = run(part, None)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_unrounded_output_and_gradients_from_it():
    """The forward's out_f32 is the output before its rounding: the bf16 out
    is its rounding bit for bit (plain and key-split kernels), and it is
    closer to the oracle's output than out is (it lacks out's own rounding,
    2^-9 relative). The backward forming D from it meets the same bound.
    (In a deep stack this matters: with values grown alike, p (dp - D) is a
    small difference and out's rounding in D comes back magnified in du,
    dvb and dR; the stack's gradient tests show it.)"""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, B=2, H=2, L=128, M=384, seed=11, valid_mode="random")
    dout = draw_dout(x["q"].shape, 11)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    valid = x["valid"].to(DEV)
    B, H, L, dh = q.shape
    ref_out = oa.rel_attn(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["r"]), f64(x["u"]),
                          f64(x["vb"]), valid=x["valid"].numpy())["out"]
    ref = oracle(x, dout)
    for splits in (1, 2):
        out = torch.empty_like(q)
        o32 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        lse = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid, lse=lse, out_f32=o32,
                             kv_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o32.to(torch.bfloat16), out), splits
        e32 = err_report(f64(o32), ref_out)["rel_norm"]
        e16 = err_report(f64(out), ref_out)["rel_norm"]
        say(f"  splits={splits}: out_f32 rel_norm {e32:.2e}, bf16 out {e16:.2e}")
        assert e32 < e16
        g = txl.txl_rel_attn_bwd(q, k, v, r, u, vb, out, lse, dout.to(DEV), {},
                                 mem_valid=valid, out_f32=o32)
        torch.cuda.synchronize()
        got = {n: f64(g[n]) for n in NAMES}
        check(got, ref, f"splits={splits} out_f32")
        hidden_rows_zero(got, x)
