"""GPU parity of txl_segment_step (the N-layer stack) against the fp64 oracle.

Every layer is checked teacher-forced: the oracle's layer n gets exactly the
GPU's bf16 input H^(n-1) and the GPU's memory of layer n-1 before the step,
and its fp64 output is compared with the GPU's H^(n). The ring contents after
the step must equal Tail_M([memory; H^(n)]) bit for bit. The free-running
end-to-end difference is printed, not gated.

Tolerance of a layer output (bf16, post-LayerNorm, unit scale):
    |gpu - ref| <= 1.5e-2 + 2^-7 |ref|
the bf16 attention figure of the method's goals plus two bf16 half-ulps of
the element's magnitude: one for the bf16 rounding of the first LayerNorm's
output, which the feed-forward residual carries to the output, and one for
the rounding of the output itself.
"""
import numpy as np
import pytest
import torch

import txl_synth
import transformer_xl_relative_txl_amd as txl
from oracle import memory as om
from oracle import stack as ost
from tests.gpu_helpers import f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL, RTOL = 1.5e-2, 2.0 ** -7
OUT_MAJOR = ("wq", "wk", "wv", "wo", "wr", "w1", "w2")


def gpu_weights(w):
    emb = w["emb"].to(DEV).contiguous()
    layers = []
    for lw in w["layers"]:
        g = {}
        for k, t in lw.items():
            g[k] = (t.t() if k in OUT_MAJOR else t).contiguous().to(DEV)
        layers.append(g)
    return emb, layers


def make_stack(cfg, w):
    emb, layers = gpu_weights(w)
    st = txl.TxlStack(n_layer=len(layers), d=cfg.d, n_head=cfg.H, d_h=cfg.d_h, d_ff=cfg.d_ff,
                      vocab=cfg.vocab, B=cfg.B, L=cfg.L, M=cfg.M, emb=emb, layers=layers)
    return st, (emb, layers)


def read_rings(mems):
    out = []
    for m in mems:
        buf = torch.empty_like(m.data)
        txl.txl_mem_read_logical(m, buf)
        out.append(buf)
    torch.cuda.synchronize()
    return [(f64(b), m.valid.cpu().numpy().copy()) for b, m in zip(out, mems)]


class Oracle:
    """Lazily converted fp64 weights and R tables of the stack."""

    def __init__(self, cfg, w):
        self.cfg, self.w = cfg, w
        self._layers, self._r = {}, {}
        self.emb = f64(w["emb"])

    def layer(self, n):
        if n not in self._layers:
            self._layers[n] = {k: f64(t) for k, t in self.w["layers"][n].items()}
        return self._layers[n]

    def r(self, n):
        if n not in self._r:
            c = self.cfg
            self._r[n] = ost.rel_pos_table(self.layer(n)["wr"], c.M, c.L, c.H, c.d_h)
        return self._r[n]

    def forward(self, n, h, mem):
        c = self.cfg
        return ost.layer_forward(h, mem, self.layer(n), self.r(n), c.M, c.H, c.d_h)


def run_stream(cfg, w, tokens, resets, check, n_layer, rows_to_check, layers_to_check,
               all_rows_layer=None):
    """Stream the segments through the GPU stack; at segments in `check`
    compare memories (all rows, all rings, bit-exact) and layer outputs
    (teacher-forced) with the oracle: rows `rows_to_check` at layers
    `layers_to_check`, and, when `all_rows_layer(s)` is given, every row at
    that layer of segment s. Returns the worst errors and the number of
    compared elements beyond 1.5e-2 absolute (the bf16 attention figure)."""
    st, keep = make_stack(cfg, w)
    orc = Oracle(cfg, w)
    M, L, B, d = cfg.M, cfg.L, cfg.B, cfg.d
    assert L <= M, "the last L ring rows hold H^(n) only when L <= M"
    mems = [txl.TxlMem.empty(B, M, d) for _ in range(n_layer + 1)]
    h_out = torch.empty((B, L, d), dtype=torch.bfloat16, device=DEV)
    worst = {"layer_abs": 0.0, "layer_excess": -1.0, "n_compared": 0, "n_over_1.5e-2": 0,
             "min_mem": M, "max_mem": 0}
    tok_d = tokens.to(DEV)
    for s in range(tokens.shape[0]):
        if resets[s].any():
            txl.txl_mem_reset_rows(mems, resets[s].to(DEV).contiguous())
        before = read_rings(mems) if s in check else None
        st.step(tok_d[s].contiguous(), mems, h_out)
        torch.cuda.synchronize()
        if s not in check:
            continue
        after = read_rings(mems)
        say(f"segment {s}: valid {[int(v) for v in before[0][1]]} before the step")
        # H^(0) is the embedding of the tokens, exactly
        emb_ref = orc.emb[tokens[s].numpy()]
        assert np.array_equal(after[0][0][:, M - L:], emb_ref)
        assert np.array_equal(f64(h_out), after[n_layer][0][:, M - L:])
        for n in range(n_layer + 1):
            data_b, valid_b = before[n]
            data_a, valid_a = after[n]
            hs = data_a[:, M - L:]          # H^(n) of this segment
            for b in range(B):
                old = data_b[b, M - valid_b[b]:]
                want = om.tail(np.concatenate([old, hs[b]], axis=0), M)
                assert valid_a[b] == want.shape[0], (s, n, b)
                assert np.array_equal(data_a[b, M - valid_a[b]:], want), (s, n, b)
        pairs = {(n, b) for n in layers_to_check for b in rows_to_check}
        if all_rows_layer is not None:
            pairs |= {(all_rows_layer(s), b) for b in range(B)}
        for n, b in sorted(pairs):          # layer n maps H^(n-1) -> H^(n), 1-based
            data_b, valid_b = before[n - 1]
            mem = data_b[b, M - valid_b[b]:]
            h_in = after[n - 1][0][b, M - L:]
            ref = orc.forward(n - 1, h_in, mem)
            got = after[n][0][b, M - L:]
            err = np.abs(got - ref)
            excess = float((err - (ATOL + RTOL * np.abs(ref))).max())
            worst["layer_abs"] = max(worst["layer_abs"], float(err.max()))
            worst["layer_excess"] = max(worst["layer_excess"], excess)
            worst["n_compared"] += int(err.size)
            worst["n_over_1.5e-2"] += int((err > ATOL).sum())
            worst["min_mem"] = min(worst["min_mem"], int(mem.shape[0]))
            worst["max_mem"] = max(worst["max_mem"], int(mem.shape[0]))
            say(f"  seg {s} layer {n} row {b} (mem {mem.shape[0]}): max abs err "
                f"{err.max():.3e}, mean {err.mean():.2e}, beyond 1.5e-2: {int((err > ATOL).sum())}")
            assert excess <= 0.0, (s, n, b, float(err.max()))
    st.close()
    del keep
    say(f"  compared {worst['n_compared']} layer-output elements, "
        f"{worst['n_over_1.5e-2']} beyond 1.5e-2 absolute, worst {worst['layer_abs']:.3e}")
    return worst


def small_cfg(M=72, L=40, B=3, seed=3):
    return txl_synth.StackConfig("tiny", "bf16", n_layer=2, d=256, H=4, d_h=64, d_ff=512,
                                 vocab=97, B=B, L=L, M=M, n_seg=5, seed=seed, w_std=0.05,
                                 reset_every=0)


def test_small_stack_stream_with_resets():
    cfg = small_cfg()
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    resets = txl_synth.reset_schedule(cfg)
    resets[3, 1] = 1
    worst = run_stream(cfg, w, tokens, resets, check=set(range(cfg.n_seg)),
                       n_layer=cfg.n_layer, rows_to_check=range(cfg.B), layers_to_check=[1, 2])
    say(f"small stack worst: {worst}")


def test_rel_pos_table_matches_oracle():
    """a1: the library's R (fp64 sinusoid, fp32 projection, bf16 result)
    against the oracle's fp64 table: within one bf16 ulp plus fp32 slack."""
    cfg = small_cfg()
    w = txl_synth.stack_weights(cfg)
    st, keep = make_stack(cfg, w)
    torch.cuda.synchronize()
    for n in range(cfg.n_layer):
        ref = ost.rel_pos_table(f64(w["layers"][n]["wr"]), cfg.M, cfg.L, cfg.H, cfg.d_h)
        ref = ref.transpose(1, 0, 2).reshape(cfg.M + cfg.L, cfg.H * cfg.d_h)
        got = f64(st.r_table(n))
        err = np.abs(got - ref)
        say(f"R layer {n}: max abs err {err.max():.3e}, max |R| {np.abs(ref).max():.3f}")
        assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-5).all()
    st.close()
    del keep


def test_rel_pos_table_fp32_entry_point():
    M, L, H, dh = 8, 4, 1, 64
    wr = (torch.randn((H * dh, H * dh), generator=torch.Generator().manual_seed(4)) / 8)
    r = torch.empty((M + L, H * dh), device=DEV)
    txl.txl_rel_pos_table(wr.to(DEV), M, L, H, dh, r)
    ref = ost.rel_pos_table(wr.t().double().numpy(), M, L, H, dh)[0]
    err = np.abs(f64(r) - ref).max() / np.abs(ref).max()
    say(f"R fp32 max rel err {err:.2e}")
    assert err <= 1e-5


def test_rel_pos_table_full_size_both_dtypes():
    """R of the 18-layer workload's layer shape (M=640, L=128, d=1024, 16
    heads of 64) against the fp64 oracle: fp32 output within 1e-5 of the
    largest entry (normwise), bf16 output within one bf16 ulp plus fp32 slack."""
    M, L, H, dh, d = 640, 128, 16, 64, 1024
    g = torch.Generator().manual_seed(9)
    wr = torch.randn((H * dh, d), generator=g) / d ** 0.5      # output-major
    ref = ost.rel_pos_table(wr.t().double().numpy(), M, L, H, dh)
    ref = ref.transpose(1, 0, 2).reshape(M + L, H * dh)
    r32 = torch.empty((M + L, H * dh), device=DEV)
    txl.txl_rel_pos_table(wr.to(DEV), M, L, H, dh, r32)
    err32 = np.abs(f64(r32) - ref).max() / np.abs(ref).max()
    wb = wr.to(torch.bfloat16)
    refb = ost.rel_pos_table(wb.t().double().numpy(), M, L, H, dh)
    refb = refb.transpose(1, 0, 2).reshape(M + L, H * dh)
    rb = torch.empty((M + L, H * dh), dtype=torch.bfloat16, device=DEV)
    txl.txl_rel_pos_table(wb.to(DEV), M, L, H, dh, rb)
    errb = np.abs(f64(rb) - refb)
    say(f"R full size: fp32 max rel err {err32:.2e}, bf16 max abs err {errb.max():.2e}")
    assert err32 <= 1e-5
    assert (errb <= 2.0 ** -8 * np.abs(refb) + 1e-5).all()


def test_reset_row_equals_fresh_stream_bitwise():
    """A row reset at segment 2 produces bit-identical outputs to the same
    row of a stream that starts fresh at segment 2."""
    cfg = small_cfg(B=2, seed=5)
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    st, keep = make_stack(cfg, w)
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    outs = []
    for s in range(5):
        if s == 2:
            txl.txl_mem_reset_rows(mems, torch.tensor([1, 0], dtype=torch.uint8, device=DEV))
        st.step(tokens[s].to(DEV).contiguous(), mems, h)
        outs.append(h.clone())
    fresh = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    for s in range(2, 5):
        st.step(tokens[s].to(DEV).contiguous(), fresh, h)
        assert torch.equal(h[0], outs[s][0]), s
        if s == 2:
            assert not torch.equal(h[1], outs[s][1])
    st.close()
    del keep


def test_checkpoint_resume_bitwise():
    """Stop after segment 2, save the rings in logical order with their valid
    counts, restore them into fresh rings (head 0) and continue: outputs are
    bit-identical to the uninterrupted stream."""
    cfg = small_cfg(B=2, M=64, L=24, seed=6)
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    st, keep = make_stack(cfg, w)
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    ref = []
    saved = None
    for s in range(5):
        st.step(tokens[s].to(DEV).contiguous(), mems, h)
        ref.append(h.clone())
        if s == 2:
            saved = []
            for m in mems:
                buf = torch.empty_like(m.data)
                txl.txl_mem_read_logical(m, buf)
                saved.append((buf.clone(), m.valid.clone()))
    restored = [txl.TxlMem(d.clone(), v.clone(), 0) for d, v in saved]
    for s in range(3, 5):
        st.step(tokens[s].to(DEV).contiguous(), restored, h)
        assert torch.equal(h, ref[s]), s
    st.close()
    del keep


def test_stack_deterministic_bitwise():
    cfg = small_cfg(seed=7)
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    st, keep = make_stack(cfg, w)
    outs = []
    for _ in range(2):
        mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
        h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
        for s in range(3):
            st.step(tokens[s].to(DEV).contiguous(), mems, h)
        outs.append(h.clone())
    assert torch.equal(outs[0], outs[1])
    st.close()
    del keep


def test_stack_rejects_bad_arguments():
    cfg = small_cfg()
    w = txl_synth.stack_weights(cfg)
    st, keep = make_stack(cfg, w)
    mems = [txl.TxlMem.empty(cfg.B, cfg.M, cfg.d) for _ in range(cfg.n_layer + 1)]
    h = torch.empty((cfg.B, cfg.L, cfg.d), dtype=torch.bfloat16, device=DEV)
    tok = torch.zeros((cfg.B, cfg.L), dtype=torch.int32, device=DEV)
    bad = mems[:-1] + [txl.TxlMem.empty(cfg.B, cfg.M + 1, cfg.d)]
    with pytest.raises(txl.TxlError) as e:
        st.step(tok, bad, h)
    assert e.value.status_name == "TXL_ERR_INVALID_ARG"
    ws = st.workspace
    st.workspace = ws[: ws.numel() // 2]
    with pytest.raises(txl.TxlError) as e:
        st.step(tok, mems, h)
    assert e.value.status_name == "TXL_ERR_WORKSPACE"
    st.workspace = ws
    assert all(m.head == 0 for m in mems)
    st.close()
    del keep


# ----------------------------------------------------------------------------
# the full-size workloads
# ----------------------------------------------------------------------------
def test_sixteen_layers_full_size():
    """16 layers, d=512, B=16, L=M=384, 8 segments streamed (full size on the
    GPU); memories checked for every row and ring at segments 0, 1, 7; every
    row teacher-forced at one layer per checked segment (16, 8, 1), rows 0
    and 15 also at layers 1, 2, 8, 16."""
    cfg = txl_synth.STACK_CONFIGS["16layer_d512"]
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    resets = txl_synth.reset_schedule(cfg)
    layer_of = {0: 16, 1: 8, 7: 1}
    worst = run_stream(cfg, w, tokens, resets, check=set(layer_of), n_layer=cfg.n_layer,
                       rows_to_check=[0, cfg.B - 1], layers_to_check=[1, 2, 8, 16],
                       all_rows_layer=layer_of.get)
    say(f"16 layers worst: {worst}")


def test_eighteen_layers_long_memory_with_resets():
    """18 layers, d=1024, B=8, L=128, M=640, 16 segments with every row
    resetting at segments 0, 4, 8, 12; checks at segments 1, 3, 4 and 15
    (memories of 128, 384, 0 and 384 states): every row at one layer per
    checked segment, rows 0 and 7 at layers 1, 9, 18."""
    cfg = txl_synth.STACK_CONFIGS["18layer_d1024"]
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    resets = txl_synth.reset_schedule(cfg)
    layer_of = {1: 18, 3: 9, 4: 5, 15: 1}
    worst = run_stream(cfg, w, tokens, resets, check=set(layer_of), n_layer=cfg.n_layer,
                       rows_to_check=[0, cfg.B - 1], layers_to_check=[1, 9, 18],
                       all_rows_layer=layer_of.get)
    say(f"18 layers worst: {worst}")


def test_eighteen_layers_steady_state_wrapped_ring():
    """The 18-layer workload's labelled steady state: 16 segments with no
    reset after the first, so from segment 5 on every layer attends over a
    full memory of 640 states and each ring has wrapped (head moves 128 per
    segment over 640 slots); this is the state the stack benchmark times.
    Checks at segments 5, 9 and 15: every ring and row bit-exact, every row
    at one layer per checked segment, rows 0 and 7 at layers 1, 9, 18."""
    cfg = txl_synth.STACK_CONFIGS["18layer_d1024"]
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg)
    resets = torch.zeros((cfg.n_seg, cfg.B), dtype=torch.uint8)
    resets[0] = 1
    layer_of = {5: 18, 9: 2, 15: 10}
    worst = run_stream(cfg, w, tokens, resets, check=set(layer_of), n_layer=cfg.n_layer,
                       rows_to_check=[0, cfg.B - 1], layers_to_check=[1, 9, 18],
                       all_rows_layer=layer_of.get)
    assert worst["min_mem"] == cfg.M, worst
    say(f"18 layers steady state worst: {worst}")


def test_eighteen_layers_staggered_resets():
    """The 18-layer workload with the staggered per-row reset schedule: row
    b resets when (s + b) mod 4 == 0, so the rows of one step hold memories
    of different lengths (0, 128, 256, 384 states side by side). Checks at
    segments 2, 5 and 9: every row at one layer, rows 0 and 7 at layers 1
    and 18."""
    cfg = txl_synth.STACK_CONFIGS["18layer_d1024"]
    w = txl_synth.stack_weights(cfg)
    tokens = txl_synth.stack_tokens(cfg, n_seg=10)
    resets = txl_synth.reset_schedule(cfg, n_seg=10, staggered=True)
    layer_of = {2: 1, 5: 12, 9: 18}
    worst = run_stream(cfg, w, tokens, resets, check=set(layer_of), n_layer=cfg.n_layer,
                       rows_to_check=[0, cfg.B - 1], layers_to_check=[1, 18],
                       all_rows_layer=layer_of.get)
    assert worst["min_mem"] == 0 and worst["max_mem"] == 384, worst
    say(f"18 layers staggered resets worst: {worst}")
