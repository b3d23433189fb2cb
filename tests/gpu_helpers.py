"""Shared helpers of the GPU parity tests (inputs, oracle calls, tolerances).

The oracle is called here on fp64 copies of exactly the values the GPU
receives; nothing computed by the HIP path ever becomes an oracle input.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import txl_synth
from oracle import attention as oa
from oracle import stack as ost

# Agreement criteria of the method's statement of goals: fp32 attention within
# 1e-5 max relative error (normwise: max|gpu - ref| / max|ref|), bf16
# attention within 1.5e-2 max absolute error on unit-scale outputs.
F32_REL_TOL = 1e-5
BF16_ABS_TOL = 1.5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def rel_table(x, cfg, M, L, H):
    """R for the attention workloads: the oracle's fp64 sinusoid projected
    by the drawn W_R, rounded to the workload dtype. The same rounded table
    goes to the GPU and to the oracle."""
    dh = cfg.d_h
    w = f64(x["w_r"])[: H * dh, : H * dh]
    r = ost.rel_pos_table(w, M, L, H, dh)
    return torch.from_numpy(r).to(txl_synth.torch_dtype(cfg.dtype))


def attn_case(cfg, B=None, L=None, M=None, H=None, seed=None, valid_mode="full"):
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    M = cfg.M if M is None else M
    H = cfg.H if H is None else H
    x = txl_synth.attn_inputs(cfg, B=B, L=L, M=M, H=H, seed=seed)
    x["r"] = rel_table(x, cfg, M, L, H)
    x["valid"] = txl_synth.valid_counts(B, M, valid_mode,
                                        seed=cfg.seed if seed is None else seed)
    return x


def oracle_attn(x, b_idx=None, h_idx=None):
    """fp64 oracle on (optionally) a subset of batch rows and heads."""
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    r, u, vb = f64(x["r"]), f64(x["u"]), f64(x["vb"])
    valid = x["valid"].numpy()
    if b_idx is not None:
        q, k, v, valid = q[b_idx], k[b_idx], v[b_idx], valid[b_idx]
    if h_idx is not None:
        q, k, v = q[:, h_idx], k[:, h_idx], v[:, h_idx]
        r, u, vb = r[h_idx], u[h_idx], vb[h_idx]
    return oa.rel_attn(q, k, v, r, u, vb, valid=valid)


def err_report(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu - ref)
    max_abs = float(d.max()) if d.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    rel_norm = max_abs / scale if scale > 0 else max_abs
    rel_elem = float((d / np.maximum(np.abs(ref), 1e-3 * scale)).max()) if d.size else 0.0
    return {"max_abs": max_abs, "rel_norm": rel_norm, "rel_elem": rel_elem}


def assert_close(dtype: str, gpu: np.ndarray, ref: np.ndarray, what: str):
    rep = err_report(gpu, ref)
    say(f"  {what}: {rep}")
    if dtype == "f32":
        assert rep["rel_norm"] <= F32_REL_TOL, (what, rep)
    else:
        assert rep["max_abs"] <= BF16_ABS_TOL, (what, rep)
    return rep
