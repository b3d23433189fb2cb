"""GPU parity of txl_rel_attn_fwd against the fp64 oracle (through the C ABI).

Cases: the 4x12 fp32 example, one bf16 layer with and without memory, the
large bf16 layer at full size (sampled heads/rows compared), ragged shapes
that leave partial tiles, partly valid memories, strided layouts, and the
bit-exact distance and mask probes.
"""
import math

import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import attention as oa
from tests.gpu_helpers import assert_close, attn_case, f64, oracle_attn, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_gpu(x, lse=False, layout="bhld"):
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    valid = x["valid"].to(DEV)
    B, H, L, dh = q.shape
    if layout == "blhd":
        # tensors stored [B, L, H, d_h] (what a projection writes), passed as views
        q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        out = torch.full((B, L, H, dh), float("nan"), dtype=q.dtype, device=DEV).permute(0, 2, 1, 3)
    else:
        out = torch.full((B, H, L, dh), float("nan"), dtype=q.dtype, device=DEV)
    lse_t = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=DEV) if lse else None
    txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid, lse=lse_t)
    torch.cuda.synchronize()
    return out, lse_t


def check(cfg, x, what, b_idx=None, h_idx=None, lse=True, layout="bhld"):
    say(f"case {what}: B,H,L,M = {tuple(x['q'].shape[:3]) + (x['k'].shape[2] - x['q'].shape[2],)}"
        f" dtype={cfg.dtype} layout={layout}")
    out, lse_t = run_gpu(x, lse=lse, layout=layout)
    ref = oracle_attn(x, b_idx, h_idx)
    g = f64(out)
    gl = f64(lse_t) if lse else None
    if b_idx is not None:
        g = g[b_idx]
        gl = gl[b_idx] if lse else None
    if h_idx is not None:
        g = g[:, h_idx]
        gl = gl[:, h_idx] if lse else None
    assert np.isfinite(g).all()
    assert_close(cfg.dtype, g, ref["out"], what + " out")
    if lse:
        # lse is fp32 on both paths; it is a log-normaliser of O(10) magnitude
        tol = 1e-5 if cfg.dtype == "f32" else 2e-2
        d = float(np.abs(gl - ref["lse"]).max())
        say(f"  {what} lse max abs err {d:.3e}")
        assert d <= tol * max(1.0, float(np.abs(ref["lse"]).max()))


def test_fp32_single_head_4x12():
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32"]
    check(cfg, attn_case(cfg), "4x12_f32")


@pytest.mark.parametrize("valid_mode", ["full", "mixed", "empty"])
def test_fp32_4x12_valid_counts(valid_mode):
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32"]
    check(cfg, attn_case(cfg, B=3, valid_mode=valid_mode), f"4x12_f32 valid={valid_mode}")


def test_bf16_layer_with_memory():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    check(cfg, attn_case(cfg), "B4_H8_L128_M128")


def test_bf16_layer_without_memory():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M0"]
    check(cfg, attn_case(cfg), "B4 H8 L128 M0")


def test_bf16_large_layer_full_size_every_slice():
    """The large layer at full size, launched whole as the benchmark launches
    it; the oracle checks every (batch row, head) slice, all 512 queries
    each (the tile dealing, XCD placement and copy workers all depend on the
    workgroup index, so no slice is left out)."""
    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    check(cfg, attn_case(cfg), "B8_H16_L512_M512")


def test_bf16_large_layer_mixed_valid_every_slice():
    """The large layer's shape with per-row valid counts (row 0 full, row 1
    empty, the rest random): every slice against the oracle."""
    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    check(cfg, attn_case(cfg, seed=21, valid_mode="mixed"), "B8_H16_L512_M512 mixed valid")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,L,M,mode", [
    (3, 2, 100, 37, "mixed"),   # ragged query and key tails
    (2, 3, 1, 0, "full"),       # one query, no memory
    (2, 2, 1, 9, "mixed"),      # one query, memory only
    (2, 1, 257, 300, "mixed"),  # M > L, several tiles, partial last
    (1, 2, 65, 1, "full"),
    (2, 2, 130, 640, "mixed"),  # long memory (M = 5L)
    (2, 2, 600, 50, "mixed"),   # five query tiles (odd count, ragged last)
    (1, 1, 1000, 24, "full"),   # eight query tiles
])
def test_ragged_shapes(dtype, B, H, L, M, mode):
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32" if dtype == "f32" else "B4_H8_L128_M128"]
    check(cfg, attn_case(cfg, B=B, H=H, L=L, M=M, seed=B * 1000 + L + M, valid_mode=mode),
          f"ragged {dtype} B{B} H{H} L{L} M{M} {mode}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_blhd_layout(dtype):
    cfg = txl_synth.ATTN_CONFIGS["4x12_f32" if dtype == "f32" else "B4_H8_L128_M128"]
    x = attn_case(cfg, B=2, H=4, L=70, M=50, seed=5, valid_mode="mixed")
    check(cfg, x, f"strided {dtype}", layout="blhd")


@pytest.mark.parametrize("B,L", [(0, 16), (2, 0)])
def test_empty_is_noop(B, L):
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    M, H, dh = 8, 2, 64
    q = torch.zeros((B, H, L, dh), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, H, M + L, dh), dtype=torch.bfloat16, device=DEV)
    r = torch.zeros((H, M + L, dh), dtype=torch.bfloat16, device=DEV)
    u = torch.zeros((H, dh), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, H, L, dh), dtype=torch.bfloat16, device=DEV)
    txl.txl_rel_attn_fwd(q, k, k, r, u, u, out)
    torch.cuda.synchronize()
    del cfg


# ----------------------------------------------------------------------------
# bit-exact probes through the public API
# ----------------------------------------------------------------------------
def _probe_tensors(B, H, L, M, dtype):
    dh = 64
    dt = txl_synth.torch_dtype(dtype)
    q = torch.zeros((B, H, L, dh), dtype=dt)
    k = torch.zeros((B, H, M + L, dh), dtype=dt)
    v = torch.zeros((B, H, M + L, dh), dtype=dt)
    for jp in range(M + L):
        v[:, :, jp, jp] = 1.0  # one-hot by logical key index
    r = torch.zeros((H, M + L, dh), dtype=dt)
    u = torch.zeros((H, dh), dtype=dt)
    return q, k, v, r, u


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_distance_probe(dtype):
    """q = e0, k = u = v = 0, R[t*] = 200 e0 (scale 1): every row's softmax
    puts all its weight on the key whose in-tile index j' + L - 1 - i is t*,
    when that key is visible; otherwise all visible scores tie at 0."""
    B, H, L, M = 2, 1, 24, 40
    valid = torch.tensor([M, 13], dtype=torch.int32)
    q, k, v, r0, u = _probe_tensors(B, H, L, M, dtype)
    q[..., 0] = 1.0
    qd, kd, vd, ud = q.to(DEV), k.to(DEV), v.to(DEV), u.to(DEV)
    vis = [oa.visible_mask(L, M, int(valid[b])) for b in range(B)]
    n_hit = 0
    for t_star in range(M + L):
        r = r0.clone()
        r[:, t_star, 0] = 200.0
        out = torch.full((B, H, L, 64), float("nan"), dtype=q.dtype, device=DEV)
        txl.txl_rel_attn_fwd(qd, kd, vd, r.to(DEV), ud, ud, out,
                             mem_valid=valid.to(DEV), scale=1.0)
        o = out.float().cpu().numpy()
        for b in range(B):
            for i in range(L):
                jp = t_star + i - (L - 1)
                if 0 <= jp < M + L and vis[b][i, jp]:
                    expect = np.zeros(64, dtype=np.float32)
                    expect[jp] = 1.0
                    assert np.array_equal(o[b, 0, i], expect), (t_star, b, i)
                    n_hit += 1
                else:
                    n = int(vis[b][i].sum())
                    sel = o[b, 0, i][: M + L][vis[b][i]]
                    np.testing.assert_allclose(sel, 1.0 / n, rtol=1e-2 if dtype == "bf16" else 1e-6)
                    assert (o[b, 0, i][: M + L][~vis[b][i]] == 0).all()
    say(f"distance probe {dtype}: {n_hit} selected rows exact")
    assert n_hit > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mask_probe(dtype):
    """All scores 0 and V one-hot by key index: row i is 1/|visible_i| on
    exactly its visible keys and exactly 0 elsewhere (column windows of 64
    keys cover M + L > 64)."""
    B, H, L, M = 3, 2, 37, 100
    valid = torch.tensor([M, 0, 41], dtype=torch.int32)
    dt = txl_synth.torch_dtype(dtype)
    dh = 64
    q = torch.zeros((B, H, L, dh), dtype=dt, device=DEV)
    k = torch.zeros((B, H, M + L, dh), dtype=dt, device=DEV)
    r = torch.zeros((H, M + L, dh), dtype=dt, device=DEV)
    u = torch.zeros((H, dh), dtype=dt, device=DEV)
    vis = np.stack([oa.visible_mask(L, M, int(valid[b])) for b in range(B)])
    for w0 in range(0, M + L, dh):
        v = torch.zeros((B, H, M + L, dh), dtype=dt)
        for jp in range(w0, min(w0 + dh, M + L)):
            v[:, :, jp, jp - w0] = 1.0
        out = torch.full((B, H, L, dh), float("nan"), dtype=dt, device=DEV)
        txl.txl_rel_attn_fwd(q, k, v.to(DEV), r, u, u, out, mem_valid=valid.to(DEV))
        o = out.float().cpu().numpy()
        w1 = min(w0 + dh, M + L)
        for b in range(B):
            n = vis[b].sum(axis=1)
            for h in range(H):
                win = o[b, h, :, : w1 - w0]
                mask = vis[b][:, w0:w1]
                assert (win[~mask] == 0).all()
                expect = np.broadcast_to((1.0 / n)[:, None], win.shape)[mask]
                np.testing.assert_allclose(win[mask], expect,
                                           rtol=1e-2 if dtype == "bf16" else 1e-6)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_deterministic_bitwise():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode="mixed")
    a, _ = run_gpu(x)
    b, _ = run_gpu(x)
    assert torch.equal(a, b)


def test_row_and_head_permutation_bitwise():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode="mixed")
    base, _ = run_gpu(x)
    pb = torch.tensor([2, 0, 3, 1])
    y = dict(x)
    for key in ("q", "k", "v", "valid"):
        y[key] = x[key][pb]
    perm, _ = run_gpu(y)
    assert torch.equal(perm, base[pb.to(DEV)])
    ph = torch.tensor([7, 1, 0, 2, 3, 4, 6, 5])
    z = dict(x)
    for key in ("q", "k", "v"):
        z[key] = x[key][:, ph]
    for key in ("r", "u", "vb"):
        z[key] = x[key][ph]
    perm_h, _ = run_gpu(z)
    assert torch.equal(perm_h, base[:, ph.to(DEV)])


def test_invalid_arguments_rejected_before_launch():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, B=1, H=1, L=8, M=8)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    out = torch.zeros_like(q)
    sentinel = out.clone()
    # misaligned q (offset by one element): unsupported, nothing written
    qq = torch.zeros(q.numel() + 8, dtype=q.dtype, device=DEV)[1:1 + q.numel()].view_as(q)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(qq, k, v, r, u, vb, out)
    assert e.value.status_name == "TXL_ERR_UNSUPPORTED"
    # d_h other than 64
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(q[..., :32], k[..., :32], v[..., :32], r[..., :32],
                             u[:, :32].contiguous(), vb[:, :32].contiguous(), out[..., :32])
    assert e.value.status_name == "TXL_ERR_UNSUPPORTED"
    # non-finite scale
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, scale=float("inf"))
    assert e.value.status_name == "TXL_ERR_INVALID_ARG"
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel)
    _ = math
