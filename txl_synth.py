"""Seeded synthetic inputs for the Transformer-XL relative-attention workloads.

This module only draws random numbers and fixes shapes. It holds none of the
method's arithmetic (no sinusoid, no projection, no attention), so both the
GPU path and the fp64 oracle can take their inputs from here without sharing
any computation.

The shapes follow the pages' workloads: segment lengths T = 64..640 and memory
M between T and 5T (robocikowo.com "Transformer-XL", glossary entries on
segment and memory length), the 4-query / 8-memory single-head example with a
4x12 score (wq-win.github.io "019 Transformer-XL", section 3, worked example),
and the batched tensor contract of zty624.github.io "Transformer-XL",
section "Batched Tensor Contract". No dataset is read: tokens are uniform
random ids standing in for WikiText-103 / enwik8 text.

Every draw is fp32 from ``torch.Generator('cpu').manual_seed(seed)`` in the
order documented on each function; bf16 workloads round those fp32 draws to
bfloat16 (round to nearest even) before either side sees them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """One layer of relative attention plus the memory update of that layer."""
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    H: int
    d_h: int
    L: int
    M: int
    seed: int
    qkv_std: float      # std of q, k, v (and of mem / h for the update)
    bias_std: float     # std of the per-head biases u and v
    wr_std: float       # std of the per-head projection W_R of the sinusoid

    @property
    def d(self) -> int:
        return self.H * self.d_h


@dataclasses.dataclass(frozen=True)
class StackConfig:
    """An N-layer stack streamed over consecutive segments."""
    name: str
    dtype: str
    n_layer: int
    d: int
    H: int
    d_h: int
    d_ff: int
    vocab: int
    B: int
    L: int
    M: int
    n_seg: int
    seed: int
    w_std: float
    reset_every: int    # 0: no resets; k: every row resets when seg % k == 0


ATTN_CONFIGS: Dict[str, AttnConfig] = {
    # 4 queries, 8 memory slots, one head: the 4x12 score of the worked example
    "4x12_f32": AttnConfig("4x12_f32", "f32", B=1, H=1, d_h=64, L=4, M=8, seed=0,
                     qkv_std=1.0 / 8, bias_std=1.0 / 8, wr_std=1.0 / 8),
    "B4_H8_L128_M128": AttnConfig("B4_H8_L128_M128", "bf16", B=4, H=8, d_h=64, L=128, M=128, seed=0,
                     qkv_std=1.0, bias_std=0.02, wr_std=512 ** -0.5),
    "B4_H8_L128_M0": AttnConfig("B4_H8_L128_M0", "bf16", B=4, H=8, d_h=64, L=128, M=0, seed=0,
                       qkv_std=1.0, bias_std=0.02, wr_std=512 ** -0.5),
    "B8_H16_L512_M512": AttnConfig("B8_H16_L512_M512", "bf16", B=8, H=16, d_h=64, L=512, M=512, seed=1,
                     qkv_std=1.0, bias_std=0.02, wr_std=1024 ** -0.5),
}

STACK_CONFIGS: Dict[str, StackConfig] = {
    "16layer_d512": StackConfig("16layer_d512", "bf16", n_layer=16, d=512, H=8, d_h=64, d_ff=2048,
                      vocab=32768, B=16, L=384, M=384, n_seg=8, seed=0,
                      w_std=0.02, reset_every=0),
    "18layer_d1024": StackConfig("18layer_d1024", "bf16", n_layer=18, d=1024, H=16, d_h=64,
                      d_ff=4096, vocab=32768, B=8, L=128, M=640, n_seg=16,
                      seed=0, w_std=0.02, reset_every=4),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(gen: torch.Generator, shape, std: float) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


# ----------------------------------------------------------------------------
# attention workloads
# ----------------------------------------------------------------------------
def attn_inputs(cfg: AttnConfig, *, B: Optional[int] = None,
                L: Optional[int] = None, M: Optional[int] = None,
                H: Optional[int] = None, seed: Optional[int] = None
                ) -> Dict[str, torch.Tensor]:
    """Draw one layer's attention + memory-update inputs (CPU tensors).

    Draw order: q [B,H,L,d_h], k [B,H,M+L,d_h], v [B,H,M+L,d_h], u [H,d_h],
    vb [H,d_h], w_r [d, H*d_h], mem [B,M,d], h [B,L,d]. Overrides of B, L, M,
    H and seed give the ragged / edge-case variants used by the tests.
    Keys are in logical order: index j' in [0, M) is memory (oldest first),
    [M, M+L) is the current segment.
    Returned tensors are already rounded to the workload dtype.
    """
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    M = cfg.M if M is None else M
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    d_h = cfg.d_h
    d = H * d_h
    g = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(cfg.dtype)
    out = {
        "q": _normal(g, (B, H, L, d_h), cfg.qkv_std),
        "k": _normal(g, (B, H, M + L, d_h), cfg.qkv_std),
        "v": _normal(g, (B, H, M + L, d_h), cfg.qkv_std),
        "u": _normal(g, (H, d_h), cfg.bias_std),
        "vb": _normal(g, (H, d_h), cfg.bias_std),
        "w_r": _normal(g, (d, H * d_h), cfg.wr_std),
        "mem": _normal(g, (B, M, d), cfg.qkv_std),
        "h": _normal(g, (B, L, d), cfg.qkv_std),
    }
    return {k: t.to(dt) for k, t in out.items()}


def valid_counts(B: int, M: int, mode: str = "full", seed: int = 0
                 ) -> torch.Tensor:
    """Per-row count of valid memory slots (int32, values in [0, M]).

    mode "full": every slot valid; "empty": none (a fresh stream or a reset);
    "mixed": row 0 full, row 1 empty, the rest uniform in [0, M].
    """
    if mode == "full":
        return torch.full((B,), M, dtype=torch.int32)
    if mode == "empty":
        return torch.zeros((B,), dtype=torch.int32)
    g = torch.Generator("cpu").manual_seed(seed + 7919)
    v = torch.randint(0, M + 1, (B,), generator=g, dtype=torch.int32)
    if B > 0:
        v[0] = M
    if B > 1:
        v[1] = 0
    return v


# ----------------------------------------------------------------------------
# stack workloads
# ----------------------------------------------------------------------------
LAYER_KEYS = ("wq", "wk", "wv", "wo", "wr", "u", "vb", "ln1_g", "ln1_b",
              "w1", "w2", "ln2_g", "ln2_b")


def stack_weights(cfg: StackConfig, *, n_layer: Optional[int] = None,
                  ln_std: float = 0.0) -> Dict[str, object]:
    """Draw the stack's weights (CPU tensors, rounded to the workload dtype).

    Math orientation: a projection ``y = x W`` stores W as [in, out].
    Draw order: emb [vocab, d], then per layer wq, wk, wv [d, H*d_h],
    wo [H*d_h, d], wr [d, H*d_h], u [H, d_h], vb [H, d_h], w1 [d, d_ff],
    w2 [d_ff, d]. LayerNorm gains are 1 and shifts 0 (not drawn), unless
    ``ln_std`` > 0: then, after all of the above, per layer ln1_g, ln1_b,
    ln2_g, ln2_b are drawn as 1 + N(0, ln_std^2), N(0, ln_std^2) (gains)
    and N(0, ln_std^2) (shifts), so that gradients see gains other than 1.
    """
    n_layer = cfg.n_layer if n_layer is None else n_layer
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    dt = torch_dtype(cfg.dtype)
    d, hd = cfg.d, cfg.H * cfg.d_h
    s = cfg.w_std
    emb = _normal(g, (cfg.vocab, d), s).to(dt)
    layers: List[Dict[str, torch.Tensor]] = []
    for _ in range(n_layer):
        lw = {
            "wq": _normal(g, (d, hd), s),
            "wk": _normal(g, (d, hd), s),
            "wv": _normal(g, (d, hd), s),
            "wo": _normal(g, (hd, d), s),
            "wr": _normal(g, (d, hd), s),
            "u": _normal(g, (cfg.H, cfg.d_h), s),
            "vb": _normal(g, (cfg.H, cfg.d_h), s),
            "w1": _normal(g, (d, cfg.d_ff), s),
            "w2": _normal(g, (cfg.d_ff, d), s),
            "ln1_g": torch.ones(d), "ln1_b": torch.zeros(d),
            "ln2_g": torch.ones(d), "ln2_b": torch.zeros(d),
        }
        layers.append(lw)
    if ln_std > 0:
        for lw in layers:
            lw["ln1_g"] = 1.0 + _normal(g, (d,), ln_std)
            lw["ln1_b"] = _normal(g, (d,), ln_std)
            lw["ln2_g"] = 1.0 + _normal(g, (d,), ln_std)
            lw["ln2_b"] = _normal(g, (d,), ln_std)
    layers = [{k: t.to(dt) for k, t in lw.items()} for lw in layers]
    return {"emb": emb, "layers": layers}


def stack_tokens(cfg: StackConfig, *, n_seg: Optional[int] = None,
                 B: Optional[int] = None, L: Optional[int] = None
                 ) -> torch.Tensor:
    """Uniform random token ids [n_seg, B, L] int32 (seed = cfg.seed + 1)."""
    n_seg = cfg.n_seg if n_seg is None else n_seg
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    g = torch.Generator("cpu").manual_seed(cfg.seed + 1)
    return torch.randint(0, cfg.vocab, (n_seg, B, L), generator=g,
                         dtype=torch.int32)


def stack_dy(cfg: StackConfig, *, B: Optional[int] = None, L: Optional[int] = None,
             seed_offset: int = 2) -> torch.Tensor:
    """A gradient arriving at the stack's output: N(0, 1) fp32 [B, L, d]
    (seed = cfg.seed + seed_offset)."""
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    g = torch.Generator("cpu").manual_seed(cfg.seed + seed_offset)
    return _normal(g, (B, L, cfg.d), 1.0)


def reset_schedule(cfg: StackConfig, n_seg: Optional[int] = None,
                   B: Optional[int] = None, staggered: bool = False
                   ) -> torch.Tensor:
    """Per-segment, per-row document-boundary flags [n_seg, B] uint8.

    Segment 0 always starts a stream. With ``reset_every = k`` every row
    resets at segments 0, k, 2k, ...; ``staggered`` resets row b when
    (s + b) mod k == 0 instead (rows at different phases).
    """
    n_seg = cfg.n_seg if n_seg is None else n_seg
    B = cfg.B if B is None else B
    r = torch.zeros((n_seg, B), dtype=torch.uint8)
    r[0, :] = 1
    k = cfg.reset_every
    if k > 0:
        for s in range(n_seg):
            for b in range(B):
                if (staggered and (s + b) % k == 0) or (not staggered and s % k == 0):
                    r[s, b] = 1
    return r
