"""GPU parity of txl_rel_attn_fwd_split (keys of a query tile split over
workgroups, partial results combined by a merge kernel) against the fp64
oracle, plus its agreement with the unsplit kernel and its argument checks.

The split changes only the fp32 order in which key tiles' contributions are
summed, so the bf16 tolerance of the unsplit kernel applies unchanged.
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from tests.gpu_helpers import BF16_ABS_TOL, assert_close, attn_case, f64, oracle_attn, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(x, kv_splits, lse=True):
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    B, H, L, dh = q.shape
    out = torch.full((B, H, L, dh), float("nan"), dtype=q.dtype, device=DEV)
    lse_t = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=DEV) if lse else None
    txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=x["valid"].to(DEV), lse=lse_t,
                         kv_splits=kv_splits)
    torch.cuda.synchronize()
    return out, lse_t


def check(x, kv_splits, what, b_idx=None, h_idx=None):
    out, lse_t = run(x, kv_splits)
    ref = oracle_attn(x, b_idx, h_idx)
    g, gl = f64(out), f64(lse_t)
    if b_idx is not None:
        g, gl = g[b_idx], gl[b_idx]
    if h_idx is not None:
        g, gl = g[:, h_idx], gl[:, h_idx]
    assert np.isfinite(g).all()
    assert_close("bf16", g, ref["out"], f"{what} splits={kv_splits} out")
    d = float(np.abs(gl - ref["lse"]).max())
    say(f"  {what} splits={kv_splits} lse max abs err {d:.2e}")
    assert d <= 2e-2


@pytest.mark.parametrize("kv_splits", [2, 3, 4, 8])
@pytest.mark.parametrize("valid_mode", ["full", "random"])
def test_layer_split(kv_splits, valid_mode):
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode=valid_mode)
    check(x, kv_splits, f"B4_H8_L128_M128 valid={valid_mode}")


@pytest.mark.parametrize("B,H,L,M,kv_splits", [(2, 3, 100, 77, 3), (1, 2, 64, 0, 8),
                                                (3, 1, 33, 200, 5), (1, 1, 1, 0, 4)])
def test_ragged_and_more_splits_than_tiles(B, H, L, M, kv_splits):
    """Partial tiles, no memory, one query; 8 splits of a single key tile
    leave seven empty splits, which the merge must ignore."""
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, B=B, H=H, L=L, M=M, seed=11, valid_mode="random")
    check(x, kv_splits, f"ragged {B}x{H} L={L} M={M}")


def test_long_memory_shape_sampled():
    """The 18-layer workload's attention shape: B=8, H=16, L=128, M=640 (16 key
    tiles per query tile, 128 query tiles in all), 4 splits; rows 0 and 7,
    heads 0 and 15 against the oracle; every output finite."""
    cfg = txl_synth.AttnConfig("long", "bf16", B=8, H=16, d_h=64, L=128, M=640, seed=2,
                               qkv_std=1.0, bias_std=0.02, wr_std=1024 ** -0.5)
    x = attn_case(cfg, valid_mode="random")
    check(x, 4, "B8 H16 L128 M640", b_idx=[0, 7], h_idx=[0, 15])


def test_split_agrees_with_unsplit():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, valid_mode="random")
    o1, l1 = run(x, 1)
    o4, l4 = run(x, 4)
    err = float((o1.float() - o4.float()).abs().max())
    say(f"split 4 vs unsplit: max abs diff {err:.2e}")
    assert err <= BF16_ABS_TOL
    assert float((l1 - l4).abs().max()) <= 1e-3


def test_split_rejects_bad_arguments():
    cfg = txl_synth.ATTN_CONFIGS["B4_H8_L128_M128"]
    x = attn_case(cfg, B=1, H=1, L=64, M=64)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    r, u, vb = x["r"].to(DEV), x["u"].to(DEV), x["vb"].to(DEV)
    out = torch.empty_like(q)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, kv_splits=0)
    assert e.value.status_name == "TXL_ERR_INVALID_ARG"
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, kv_splits=2,
                             workspace=torch.empty(64, dtype=torch.uint8, device=DEV))
    assert e.value.status_name == "TXL_ERR_WORKSPACE"
    qf, kf, vf = q.float(), k.float(), v.float()
    with pytest.raises(txl.TxlError) as e:
        txl.txl_rel_attn_fwd(qf, kf, vf, r.float(), u.float(), vb.float(), torch.empty_like(qf),
                             kv_splits=2)
    assert e.value.status_name == "TXL_ERR_UNSUPPORTED"
