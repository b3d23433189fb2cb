#!/usr/bin/env python3
"""Throughput of the Transformer-XL relative-attention step on one MI355X.

Workload (a step): one layer of relative-position memory attention plus that
layer's FIFO memory update, bf16, B=8, H=16, d_h=64 (d=1024), segment L=512,
memory M=512 fully valid. Inputs are seeded synthetic tensors of that shape,
resident in HBM before timing starts; the relative-position table R (a
function of the weights and of M, L only) is built once by the library
before timing. Each timed step is txl_rel_attn_fwd_mem_update: the
attention, masked by the ring's valid counts, and the append of the segment
to that ring, in one launch; the step rotates over 32 ring/segment buffer
pairs (537 MB) so that the append is not served from the 256 MB last-level
cache. The same step as two launches (txl_rel_attn_fwd, then txl_mem_update)
and each of those alone are timed as well.

Prints one JSON line. `value` is attention TFLOP/s over the whole step
(algorithmic flops: 6*d_h per visible (query, key) pair, masked pairs not
counted). Every figure replays a captured HIP graph of K launches between
two HIP events on the launch stream; per-kernel figures come from graphs that
hold only that kernel. Before each figure the same graph is replayed back to
back, untimed, for at least SETTLE_MS of GPU time (independent of --warmup),
so the timed regions start with settled clocks; each figure is the median of
TIMED_REPEATS timed replays of exactly K steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rel-pos memory attention TFLOP/s (% bf16 MFMA peak) + mem-update GB/s, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
N_RING_SETS = 32   # rotating ring / segment pairs: 537 MB, past the 256 MB last-level cache twice
# untimed back-to-back replays before every timed figure (GPU time, ms)
SETTLE_MS = 150.0
# timed replays of K steps per figure; the median is reported
TIMED_REPEATS = 5

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by the
# same counters' reading of a plain copy of known size), valid only for the
# kernel source they were taken on.
ATTN_TRAFFIC = {"source_sha1": "c5fc50ea69f27a4d5908780d34fbfb51d4dd27d4",
                "profile": "profiles/rel_attn_B8_H16_L512_M512_hbm_traffic.md",
                "rel_attn_mfma_append_kernel": 69.34e6, "rel_attn_mfma_kernel": 52.53e6}


def attn_flops(B, H, L, M_eff, d_h):
    pairs = B * (L * M_eff + L * (L + 1) // 2)
    return 6.0 * d_h * H * pairs


def attn_hbm_bytes(B, H, L, M, d_h):
    """Algorithmic bf16 bytes of one attention launch with every memory slot
    valid: q, k, v and R read once, out written once."""
    return 2.0 * d_h * (2 * B * H * L + 2 * B * H * (M + L) + H * (M + L))


def _oracle_slices_worker(args):
    """Run the fp64 oracle on whole (batch row, head) slices, cycling over the
    given slices until `seconds` pass; returns (slices done, flops, seconds).
    Runs in a fresh process with its math libraries held to one thread."""
    slices, L, M, d_h, seconds = args
    import time as _t

    from threadpoolctl import threadpool_limits

    from oracle import attention as oa
    done, flops = 0, 0.0
    t0 = _t.perf_counter()
    with threadpool_limits(limits=1):
        while _t.perf_counter() - t0 < seconds:
            q, k, v, r, u, vb = slices[done % len(slices)]
            oa.rel_attn(q, k, v, r, u, vb, valid=[M])
            done += 1
            flops += attn_flops(1, 1, L, M, d_h)
    return done, flops, _t.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, cfg, seconds: float):
    """Time the fp64 oracle as it stands on a bounded sample of the same
    workload: whole (batch row, head) slices, all queries each. Two runs:
    one process with one math-library thread, and one process per available
    core (os.sched_getaffinity, at most 16), each with one thread, on
    disjoint slices, for `seconds` each; the oracle's rate is the sum."""
    import multiprocessing as mp

    import numpy as np

    from oracle import stack as ost

    r = ost.rel_pos_table(x["w_r"].double().numpy(), cfg.M, cfg.L, cfg.H, cfg.d_h)
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    u, vb = x["u"].double().numpy(), x["vb"].double().numpy()
    order = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]

    def piece(b, h):
        return (q[b:b + 1, h:h + 1].copy(), k[b:b + 1, h:h + 1].copy(),
                v[b:b + 1, h:h + 1].copy(), r[h:h + 1].copy(), u[h:h + 1].copy(),
                vb[h:h + 1].copy())

    cores = min(16, len(os.sched_getaffinity(0)))
    ctx = mp.get_context("spawn")     # fresh interpreters: no GPU state in the workers
    runs = {}
    for n_proc in sorted({1, cores}):
        parts = []
        for w in range(n_proc):
            mine = order[w::n_proc][:max(1, 48 // n_proc)]
            parts.append(([piece(b, h) for b, h in mine], cfg.L, cfg.M, cfg.d_h, seconds))
        with ctx.Pool(n_proc) as pool:
            res = pool.map(_oracle_slices_worker, parts)
        done = sum(d for d, _, _ in res)
        flops = sum(f for _, f, _ in res)
        el = max(e for _, _, e in res)
        runs[n_proc] = {"value": flops / el / 1e12, "slices": done, "seconds": round(el, 1)}
    best = runs[cores]
    return {"value": best["value"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle rel-attn on {best['slices']} whole (batch row, head) slices "
                      f"of the same workload ({cfg.B * cfg.H} slices per step, all {cfg.L} "
                      f"queries each) in {best['seconds']} s: {cores} processes x 1 thread",
            "one_thread": {"value": runs[1]["value"], "slices": runs[1]["slices"],
                           "seconds": runs[1]["seconds"]},
            "threads_per_process": 1, "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model()}


def stack_flops(c, m_eff, kv=False):
    """Algorithmic flops of one segment step with m_eff valid memory states:
    the Q, K/V (over m_eff + L rows; over the L new rows only when memory is
    kept projected), W^O and feed-forward products, plus the attention's
    three contractions over visible pairs. R is built once per stack and is
    not counted."""
    hd = c.H * c.d_h
    rows = c.B * c.L
    kv_rows = c.B * c.L if kv else c.B * (m_eff + c.L)
    per_layer = (2 * rows * c.d * hd + 4 * kv_rows * c.d * hd
                 + 2 * rows * hd * c.d + 4 * rows * c.d * c.d_ff
                 + attn_flops(c.B, c.H, c.L, m_eff, c.d_h))
    return c.n_layer * per_layer


def stack_train_flops(c, m_eff):
    """Algorithmic flops of one training step: the forward (stack_flops) and
    the backward: per dense product C = A W its two gradients dA = dC W^T and
    dW = A^T dC, except that dA of the K/V projection covers the segment rows
    only (the memory is a stop-gradient input), the W_R gradient through
    R = S W_R^T, and the attention backward (16 d_h per visible pair)."""
    hd = c.H * c.d_h
    rows = c.B * c.L
    kv_rows = c.B * (m_eff + c.L)
    ml = m_eff + c.L
    dw = (2 * rows * c.d * hd + 4 * kv_rows * c.d * hd + 2 * rows * hd * c.d
          + 4 * rows * c.d * c.d_ff + 2 * ml * c.d * hd)
    dx = 2 * rows * c.d * hd + 4 * rows * c.d * hd + 2 * rows * hd * c.d + 4 * rows * c.d * c.d_ff
    attn_b = attn_flops(c.B, c.H, c.L, m_eff, c.d_h) * 8.0 / 3.0
    return stack_flops(c, m_eff) + c.n_layer * (dw + dx + attn_b)


def stack_train_bench(name: str, steps: int, warmup: int) -> dict:
    """One training step of the stack with a full memory: the recording
    forward (txl_segment_step_train, rings advanced) and the segment
    backward (txl_segment_backward: every weight gradient, the embedding
    gradient), for a fixed gradient at the output, captured once as a HIP
    graph and replayed `steps` times between events."""
    import torch

    import txl_synth
    import transformer_xl_relative_txl_amd as txl

    c = txl_synth.STACK_CONFIGS[name]
    dev = torch.device("cuda:0")
    w = txl_synth.stack_weights(c, ln_std=0.1)
    out_major = ("wq", "wk", "wv", "wo", "wr", "w1", "w2")
    emb = w["emb"].to(dev).contiguous()
    layers = [{k: (t.t() if k in out_major else t).contiguous().to(dev) for k, t in lw.items()}
              for lw in w["layers"]]
    st = txl.TxlStack(n_layer=c.n_layer, d=c.d, n_head=c.H, d_h=c.d_h, d_ff=c.d_ff,
                      vocab=c.vocab, B=c.B, L=c.L, M=c.M, emb=emb, layers=layers)
    tokens = txl_synth.stack_tokens(c).to(dev)
    dy = txl_synth.stack_dy(c).to(dev).contiguous()
    h = torch.empty((c.B, c.L, c.d), dtype=torch.bfloat16, device=dev)
    mems = [txl.TxlMem.empty(c.B, c.M, c.d, device=dev) for _ in range(c.n_layer + 1)]
    tape = st.new_tape()
    grads = st.new_grads()

    def step(i):
        st.step_train(tokens[i % c.n_seg].contiguous(), mems, h, tape)
        st.backward(tape, dy, grads)

    s = 0
    while int(mems[0].valid.min().item()) < c.M or s < warmup:   # fill the memory
        step(s)
        s += 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(0)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(int(SETTLE_MS / max(e0.elapsed_time(e1), 1e-3)) + 1):   # settle the clocks
        g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = stack_train_flops(c, c.M)
    tape_mb = tape.numel() / 1e6
    ws_mb = st._bwd_ws.numel() / 1e6
    st.close()
    tflops = fl / (ms * 1e-3) / 1e12
    return {"metric": "training step TFLOP/s (N-layer stack forward + segment backward), 1 GPU",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{c.n_layer}-layer stack training step, d={c.d} H={c.H} "
                                   f"d_ff={c.d_ff} B={c.B} L={c.L} M={c.M} (memory full, "
                                   "stop-gradient; all weight and embedding gradients)",
                       "tokens_per_s": round(c.B * c.L / (ms * 1e-3), 1),
                       "tape_MB": round(tape_mb, 1), "backward_workspace_MB": round(ws_mb, 1)},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": None},
            "gflop_per_step": round(fl / 1e9, 2)}


def stack_bench(name: str, steps: int, warmup: int, kv: bool = False) -> dict:
    """One segment step of the stack with a full memory (steady state),
    captured once as a HIP graph and replayed `steps` times between events.
    With kv, memory is kept as projected keys / values (txl_segment_step_kv,
    capacity 2M + L): the graph holds one whole period of the window (the
    steps from one compaction to the next, the compaction included) and the
    time is per segment."""
    import torch

    import txl_synth
    import transformer_xl_relative_txl_amd as txl

    c = txl_synth.STACK_CONFIGS[name]
    dev = torch.device("cuda:0")
    w = txl_synth.stack_weights(c)
    out_major = ("wq", "wk", "wv", "wo", "wr", "w1", "w2")
    emb = w["emb"].to(dev).contiguous()
    layers = [{k: (t.t() if k in out_major else t).contiguous().to(dev) for k, t in lw.items()}
              for lw in w["layers"]]
    st = txl.TxlStack(n_layer=c.n_layer, d=c.d, n_head=c.H, d_h=c.d_h, d_ff=c.d_ff,
                      vocab=c.vocab, B=c.B, L=c.L, M=c.M, emb=emb, layers=layers)
    tokens = txl_synth.stack_tokens(c).to(dev)
    h = torch.empty((c.B, c.L, c.d), dtype=torch.bfloat16, device=dev)
    if kv:
        cap = st.kv_min_capacity()
        state = [txl.TxlKVCache.empty(c.B, cap, c.H * c.d_h, device=dev)
                 for _ in range(c.n_layer)]
        period = (cap - c.M - c.L) // c.L + 1

        def step(i):
            st.step_kv(tokens[i % c.n_seg].contiguous(), state, h)
    else:
        period = 1
        state = [txl.TxlMem.empty(c.B, c.M, c.d, device=dev) for _ in range(c.n_layer + 1)]

        def step(i):
            st.step(tokens[i % c.n_seg].contiguous(), state, h)
    s = 0
    while int(state[0].valid.min().item()) < c.M or s < warmup:   # fill the memory
        step(s)
        s += 1
    if kv:
        while state[0].start != 0:          # start the captured period at the buffer front
            step(s)
            s += 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(period):
            step(i)
    if kv:
        assert state[0].start == 0
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(int(SETTLE_MS / max(e0.elapsed_time(e1), 1e-3)) + 1):   # settle the clocks
        g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (steps * period)
    fl = stack_flops(c, c.M, kv)
    st.close()
    tflops = fl / (ms * 1e-3) / 1e12
    form = ("memory kept as projected K/V, capacity 2M+L, compactions included"
            if kv else "memory kept as hidden states, re-projected every segment")
    return {"metric": "segment step TFLOP/s (N-layer stack, steady-state memory), 1 GPU",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{c.n_layer}-layer stack segment step, d={c.d} H={c.H} "
                                   f"d_ff={c.d_ff} B={c.B} L={c.L} M={c.M} (memory full; "
                                   f"{form})",
                       "tokens_per_s": round(c.B * c.L / (ms * 1e-3), 1)},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": None},
            "gflop_per_step": round(fl / 1e9, 2)}


def loss_bench(steps: int, warmup: int) -> dict:
    """Segment loss of the 16-layer workload: 16 x 384 tokens, d = 512,
    vocabulary 32768 (tied embedding), as a replayed graph of txl_lm_loss."""
    import torch

    import transformer_xl_relative_txl_amd as txl

    dev = torch.device("cuda:0")
    n_tok, d, vocab = 16 * 384, 512, 32768
    g = torch.Generator().manual_seed(0)
    h = torch.randn((n_tok, d), generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn((vocab, d), generator=g) * 0.02).to(torch.bfloat16).to(dev)
    tg = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32).to(dev)
    nll = torch.empty(n_tok, dtype=torch.float32, device=dev)
    ws = torch.empty(txl.lib().txl_lm_loss_workspace_bytes(n_tok, vocab), dtype=torch.uint8,
                     device=dev)
    for _ in range(max(1, warmup)):
        txl.txl_lm_loss(h, w, tg, nll, workspace=ws)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        txl.txl_lm_loss(h, w, tg, nll, workspace=ws)
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = 2.0 * n_tok * vocab * d
    tflops = fl / (ms * 1e-3) / 1e12
    return {"metric": "segment loss TFLOP/s (logits + log-softmax + NLL, logits never stored), 1 GPU",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"segment loss, {n_tok} tokens (16 x 384), d={d}, "
                                   f"vocab={vocab}",
                       "tokens_per_s": round(n_tok / (ms * 1e-3), 1)},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": None},
            "gflop_per_step": round(fl / 1e9, 2)}


def bwd_bench(steps: int, warmup: int) -> dict:
    """Gradients of the relative attention at the attention workload's shape
    (B=8, H=16, d_h=64, L=512, M=512 fully valid): one txl_rel_attn_bwd call
    per step (score recompute, p/g, five contractions, bias sums), replayed
    as a captured graph; forward outputs and the incoming gradient are
    resident before timing."""
    import torch

    import txl_synth
    import transformer_xl_relative_txl_amd as txl

    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    B, H, L, M, dh = cfg.B, cfg.H, cfg.L, cfg.M, cfg.d_h
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = txl_synth.attn_inputs(cfg)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    u, vb = x["u"].to(dev), x["vb"].to(dev)
    valid = torch.full((B,), M, dtype=torch.int32, device=dev)
    w_r = x["w_r"].t().contiguous().to(dev)
    r_flat = torch.empty((M + L, H * dh), dtype=torch.bfloat16, device=dev)
    txl.txl_rel_pos_table(w_r, M, L, H, dh, r_flat)
    r = r_flat.view(M + L, H, dh).permute(1, 0, 2)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid, lse=lse)
    g = torch.Generator("cpu").manual_seed(cfg.seed + 200)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(dev)
    grads: dict = {}
    ws = torch.empty(txl.txl_rel_attn_bwd_workspace_bytes(B, H, L, M), dtype=torch.uint8, device=dev)

    def bwd():
        txl.txl_rel_attn_bwd(q, k, v, r, u, vb, out, lse, dout, grads, mem_valid=valid, workspace=ws)

    for _ in range(max(1, warmup)):
        bwd()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(steps):
            bwd()
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = attn_flops(B, H, L, M, dh) * 8.0 / 3.0
    tflops = fl / (ms * 1e-3) / 1e12
    return {"metric": "relative attention backward TFLOP/s (dq, dk, dv, dR, du, dv-bias), 1 GPU",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"relative attention gradients, B={B} H={H} d_h={dh} L={L} M={M}",
                       "flops_counted": "16*d_h per visible pair: 2 score contractions "
                                        "recomputed + 6 gradient contractions",
                       "workspace_MB": round(ws.numel() / 1e6, 1)},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": None, "scope": "whole backward call"},
            "gflop_per_step": round(fl / 1e9, 2)}


def mem_sweep_bench(steps: int) -> dict:
    """The single-ring update (txl_mem_update of one ring) at segment sizes
    moving 4 to 134 MB per launch: B=8, d=1024 bf16, L = M = 128 .. 4096
    (every slot replaced), each size rotating over ring / segment pairs that
    span at least 1 GiB (cold last-level cache), replayed as a captured graph
    of `steps` launches after a settle; the median of five timed replays."""
    import torch

    import transformer_xl_relative_txl_amd as txl

    dev = torch.device("cuda:0")
    B, d = 8, 1024
    rows = []
    for L in (128, 256, 512, 1024, 2048, 4096):
        moved = 2.0 * B * L * d * 2
        n_sets = max(4, int((1 << 30) // moved) + 1)
        rings = [txl.TxlMem(torch.zeros((B, L, d), dtype=torch.bfloat16, device=dev),
                            torch.full((B,), L, dtype=torch.int32, device=dev), 0)
                 for _ in range(n_sets)]
        segs = [torch.ones((B, L, d), dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]

        def upd(i):
            txl.txl_mem_update([rings[i % n_sets]], [segs[i % n_sets]])

        for i in range(n_sets):
            upd(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                upd(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        for _ in range(int(SETTLE_MS / max(e0.elapsed_time(e1), 1e-3)) + 1):
            g.replay()
        reps = []
        for _ in range(TIMED_REPEATS):
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / steps)
        ms = sorted(reps)[len(reps) // 2]
        gbps = moved / (ms * 1e-3) / 1e9
        rows.append({"L": L, "MB_per_launch": round(moved / 1e6, 1), "us": round(ms * 1e3, 2),
                     "GB_per_s": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "rotating_MB": round(n_sets * moved / 1e6)})
        del rings, segs, g
        torch.cuda.empty_cache()
    return {"metric": "single-ring memory update GB/s by size (cold cache), 1 GPU",
            "value": rows[2]["GB_per_s"], "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": 0, "ms_per_step": rows[2]["us"] / 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "txl_mem_update of one ring [8, L, 1024], L = M, value at "
                                   "L = 512 (16.8 MB)"},
            "sweep": rows}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of each of the two oracle CPU baseline runs (0 skips them)")
    ap.add_argument("--stack", choices=["16layer_d512", "18layer_d1024"], default=None,
                    help="measure the N-layer segment step instead (16-layer d=512 "
                         "workload or 18-layer d=1024 long-memory workload)")
    ap.add_argument("--kv", action="store_true",
                    help="with --stack: keep memory as projected keys / values")
    ap.add_argument("--train", action="store_true",
                    help="with --stack: the training step (recording forward + segment backward)")
    ap.add_argument("--loss", action="store_true",
                    help="measure the segment loss (logits + cross entropy) instead")
    ap.add_argument("--bwd", action="store_true",
                    help="measure the attention gradients (txl_rel_attn_bwd) instead")
    ap.add_argument("--mem-sweep", action="store_true",
                    help="measure the single-ring update at 4 to 134 MB per launch instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not run. The step shards "
              "over batch rows with no communication: each GPU would run this benchmark on "
              "its own rows, and the job's rate is the sum.", file=sys.stderr)
        return 2

    if args.loss:
        print(json.dumps(loss_bench(args.steps, args.warmup)), flush=True)
        return 0
    if args.bwd:
        print(json.dumps(bwd_bench(args.steps, args.warmup)), flush=True)
        return 0
    if args.mem_sweep:
        print(json.dumps(mem_sweep_bench(args.steps)), flush=True)
        return 0
    if args.stack and args.train:
        print(json.dumps(stack_train_bench(args.stack, args.steps, args.warmup)), flush=True)
        return 0
    if args.stack:
        print(json.dumps(stack_bench(args.stack, args.steps, args.warmup, args.kv)), flush=True)
        return 0

    import torch

    import txl_synth
    import transformer_xl_relative_txl_amd as txl

    cfg = txl_synth.ATTN_CONFIGS["B8_H16_L512_M512"]
    B, H, L, M, dh = cfg.B, cfg.H, cfg.L, cfg.M, cfg.d_h
    d = H * dh
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = txl_synth.attn_inputs(cfg)

    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    u, vb = x["u"].to(dev), x["vb"].to(dev)
    valid = torch.full((B,), M, dtype=torch.int32, device=dev)
    w_r = x["w_r"].t().contiguous().to(dev)            # output-major [H*d_h, d]
    r_flat = torch.empty((M + L, H * dh), dtype=torch.bfloat16, device=dev)
    txl.txl_rel_pos_table(w_r, M, L, H, dh, r_flat)
    r = r_flat.view(M + L, H, dh).permute(1, 0, 2)      # [H, M+L, d_h] view
    out = torch.empty_like(q)

    g = torch.Generator("cpu").manual_seed(cfg.seed + 100)
    rings, segs = [], []
    for s in range(N_RING_SETS):
        mem = x["mem"] if s == 0 else torch.randn((B, M, d), generator=g).to(torch.bfloat16)
        rings.append(txl.TxlMem(mem.to(dev).contiguous(),
                                torch.full((B,), M, dtype=torch.int32, device=dev), 0))
        hs = x["h"] if s == 0 else torch.randn((B, L, d), generator=g).to(torch.bfloat16)
        segs.append(hs.to(dev).contiguous())

    ws = txl.txl_rel_attn_mem_update_workspace(B, device=dev)  # the fused call's counters

    def step(i):
        ring = rings[i % N_RING_SETS]
        txl.txl_rel_attn_fwd_mem_update(q, k, v, r, u, vb, out, ring, segs[i % N_RING_SETS], ws,
                                        mem_valid=ring.valid)

    def attn():
        txl.txl_rel_attn_fwd(q, k, v, r, u, vb, out, mem_valid=valid)

    def mem(i):
        txl.txl_mem_update([rings[i % N_RING_SETS]], [segs[i % N_RING_SETS]])

    for i in range(2 * N_RING_SETS):  # first touch of every buffer
        step(i)
        attn()
        mem(i)
    torch.cuda.synchronize()

    # Each figure replays a captured HIP graph of K launches on this stream:
    # no host launch gaps inside the timed regions. (A replayed ring update
    # writes the slots its capture saw; the bytes moved are the same.)
    K = args.steps

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i)
        return g

    # all layers' rings of the 16-layer stack (d=512, B=16, L=M=384) in one
    # launch: 17 rings x 12.6 MB, two rotating sets (428 MB)
    sc = txl_synth.STACK_CONFIGS["16layer_d512"]
    n_rings = sc.n_layer + 1
    multi = []
    for _s in range(2):
        mr = [txl.TxlMem(torch.zeros((sc.B, sc.M, sc.d), dtype=torch.bfloat16, device=dev),
                         torch.full((sc.B,), sc.M, dtype=torch.int32, device=dev), 0)
              for _ in range(n_rings)]
        mh = [torch.randn((sc.B, sc.L, sc.d), generator=g).to(torch.bfloat16).to(dev)
              for _ in range(n_rings)]
        multi.append((mr, mh))
    multi_bytes = 2.0 * n_rings * sc.B * min(sc.L, sc.M) * sc.d * 2

    def mem_multi(i):
        mr, mh = multi[i % 2]
        txl.txl_mem_update(mr, mh)

    for i in range(2):
        mem_multi(i)
    # Every graph is captured first: capturing leaves the GPU idle long
    # enough for its clocks to drop, which a timed replay right after would
    # pay for.
    g_step = capture(step)
    g_sep = capture(lambda i: (attn(), mem(i)))
    g_attn = capture(lambda i: attn())
    g_mem = capture(lambda i: mem(i))
    g_multi = capture(mem_multi)
    # W untimed warmup steps (as passed), replayed from a graph
    if args.warmup > 0:
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm):
            for i in range(args.warmup):
                step(i)
        g_warm.replay()
        torch.cuda.synchronize()

    def settle(g, ms):
        """Replay g back to back for at least `ms` of GPU time, untimed: a
        cold or idle GPU needs tens of ms of continuous work before its
        clocks settle, whatever the warm-up count."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        once = max(e0.elapsed_time(e1), 1e-3)
        n = max(1, int(ms / once + 0.999))
        for _ in range(n):
            g.replay()
        torch.cuda.synchronize()
        return once * (n + 1)

    def timed(g, settle_ms=SETTLE_MS):
        """Settle, then TIMED_REPEATS timed replays of exactly K steps, each
        between a synchronize and two HIP events on the launch stream; the
        figure is their median (a rare multi-microsecond stall of the device
        lands in one repeat, not in the figure), all repeats are reported."""
        settled = settle(g, settle_ms)
        reps, walls = [], []
        for _ in range(TIMED_REPEATS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t = time.perf_counter()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t)
            reps.append(e0.elapsed_time(e1) / K)
        order = sorted(range(len(reps)), key=lambda j: reps[j])
        mid = order[len(order) // 2]
        return reps[mid], walls[mid], settled, reps

    step_ms, wall, settled_ms, step_reps = timed(g_step)
    sep_ms = timed(g_sep)[0]
    attn_ms = timed(g_attn)[0]
    mem_ms = timed(g_mem)[0]
    multi_ms = timed(g_multi)[0]

    import hashlib
    src = os.path.join(ROOT, "transformer_xl_relative_txl_amd", "csrc", "rel_attn_mfma.hip")
    with open(src, "rb") as fh:
        same_kernel = hashlib.sha1(fh.read()).hexdigest() == ATTN_TRAFFIC["source_sha1"]
    traffic = ATTN_TRAFFIC["rel_attn_mfma_append_kernel"] if same_kernel else None
    attn_traffic = ATTN_TRAFFIC["rel_attn_mfma_kernel"] if same_kernel else None
    traffic_src = (f"not measured by this run: rocprofv3 FETCH_SIZE and WRITE_SIZE of this "
                   f"kernel source (sha1 {ATTN_TRAFFIC['source_sha1'][:12]}), scaled by the "
                   f"same counters' reading of a plain copy; {ATTN_TRAFFIC['profile']}"
                   if same_kernel else "null: the kernel source differs from the profiled one")

    flops = attn_flops(B, H, L, M, dh)
    attn_bytes = attn_hbm_bytes(B, H, L, M, dh)
    Lp = min(L, M)
    mem_bytes = 2.0 * B * Lp * d * 2
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    mem_gbps = mem_bytes / (mem_ms * 1e-3) / 1e9
    value = flops / (step_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one layer rel-attn + mem update, B=8 H=16 d_h=64 L=512 M=512",
                   "B": B, "H": H, "d_h": dh, "L": L, "M": M, "valid": M,
                   "seed": cfg.seed},
        # the step's one launch: the attention with the ring append in its shadow
        "roofline": {"kernel": "rel_attn_mfma_append_kernel", "bound": "mfma",
                     "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "algorithmic_bytes": round(attn_bytes + mem_bytes)},
        "settle_ms_before_each_figure": round(settled_ms, 1),
        "ms_per_step_repeats": [round(x, 5) for x in step_reps],
        "step_two_launches_ms": round(sep_ms, 5),
        "attention_alone": {"kernel": "rel_attn_mfma_kernel", "ms": round(attn_ms, 5),
                            "achieved": round(attn_tflops, 2), "unit": "TFLOP/s",
                            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                            "traffic": attn_traffic, "algorithmic_bytes": round(attn_bytes)},
        "mem_update": {"bound": "hbm", "achieved": round(mem_gbps, 1), "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": round(mem_gbps / PEAK_HBM_GBPS, 4),
                       "bytes_per_launch": mem_bytes, "ms": round(mem_ms, 5)},
        "mem_update_all_layers": {
            "workload": "17 rings [16, 384, 512] bf16, L=384, one launch",
            "achieved": round(multi_bytes / (multi_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac": round(multi_bytes / (multi_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "bytes_per_launch": multi_bytes, "ms": round(multi_ms, 5)},
        "attn_ms": round(attn_ms, 5),
        "attn_gflop_per_launch": round(flops / 1e9, 3),
        "wall_s_timed": round(wall, 4),
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(x, cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
