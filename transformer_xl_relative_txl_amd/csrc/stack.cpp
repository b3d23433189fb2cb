// N-layer stack: one segment per call, memory rings updated in place.
//
// Order of one layer n ([P2] "019 Transformer-XL", section 3 pseudo-code):
// Q from H^(n-1), K/V from [ring n-1 in logical order; H^(n-1)], relative
// attention with ring n-1's valid counts, then ring n-1 takes H^(n-1). The
// ring is updated only after the K/V projection has read it and after the
// attention has read its valid counts: the slots being overwritten hold the
// oldest keys of this very layer ([P2] section 2: layer n reads the states
// layer n-1 produced for the previous segment).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "txl.h"
#include "txl_internal.h"

struct txl_stack {
  txl_stack_config cfg;
  const void *emb;
  std::vector<txl_layer_weights> layers;
  void *persistent;
  size_t r_bytes;  // one layer's R table
};

namespace txl {
namespace {

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

txl_status check_config(const txl_stack_config *c) {
  if (!c) return fail(TXL_ERR_INVALID_ARG, "stack: null config");
  if (c->dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "stack: only bf16 is built");
  if (c->n_layer < 1 || c->d < 1 || c->n_head < 1 || c->d_h < 1 || c->d_ff < 1 ||
      c->vocab < 1 || c->B < 1 || c->L < 1 || c->M < 0)
    return fail(TXL_ERR_INVALID_ARG, "stack: sizes must be positive (M >= 0)");
  if (c->d_h != 64) return fail(TXL_ERR_UNSUPPORTED, "stack: d_h = %d, only 64 is built", c->d_h);
  const int64_t hd = static_cast<int64_t>(c->n_head) * c->d_h;
  if (c->d % 256 || c->d_ff % 256 || hd % 128 || c->d > 4096)
    return fail(TXL_ERR_UNSUPPORTED,
                "stack: needs d and d_ff multiples of 256, H*d_h a multiple of 128, d <= 4096");
  if (!(c->ln_eps >= 0.0f) || !std::isfinite(c->ln_eps))
    return fail(TXL_ERR_INVALID_ARG, "stack: ln_eps must be finite and >= 0");
  const int64_t krows = static_cast<int64_t>(c->B) * (static_cast<int64_t>(c->M) + c->L);
  int64_t widest = c->d_ff > hd ? c->d_ff : hd;
  if (2 * hd > widest) widest = 2 * hd;
  if (c->d > widest) widest = c->d;
  if (krows * widest >= (int64_t(1) << 31) || static_cast<int64_t>(c->vocab) * c->d >= (int64_t(1) << 40))
    return fail(TXL_ERR_UNSUPPORTED, "stack: tensors too large for 32-bit row indexing");
  return TXL_OK;
}

struct WsLayout {
  size_t hc, hn, q, k, v, o, x, h1, f, total;
};

WsLayout layout(const txl_stack_config &c) {
  const size_t hd = static_cast<size_t>(c.n_head) * c.d_h;
  const size_t rows = static_cast<size_t>(c.B) * c.L;
  const size_t krows = static_cast<size_t>(c.B) * (c.M + c.L);
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  w.hc = take(rows * c.d * 2);
  w.hn = take(rows * c.d * 2);
  w.q = take(rows * hd * 2);
  w.k = take(krows * hd * 2);
  w.v = take(krows * hd * 2);
  w.o = take(rows * hd * 2);
  w.x = take(rows * c.d * 4);
  w.h1 = take(rows * c.d * 2);
  w.f = take(rows * static_cast<size_t>(c.d_ff) * 2);
  w.total = off;
  return w;
}

GemmParams dense(const void *a, int64_t lda, int rows, int N, int K, const void *w, void *c,
                 int64_t ldc) {
  GemmParams p = {};
  p.rows = rows;
  p.N = N;
  p.K = K;
  p.a = static_cast<const __bf16 *>(a);
  p.lda = lda;
  p.w0 = static_cast<const __bf16 *>(w);
  p.w1 = nullptr;
  p.n_split = N;
  p.c0 = c;
  p.c1 = nullptr;
  p.ldc = ldc;
  return p;
}

}  // namespace
}  // namespace txl

using namespace txl;

extern "C" {

TXL_API size_t txl_stack_persistent_bytes(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  const size_t hd = static_cast<size_t>(c->n_head) * c->d_h;
  return static_cast<size_t>(c->n_layer) * align256(static_cast<size_t>(c->M + c->L) * hd * 2);
}

TXL_API size_t txl_segment_step_workspace_bytes(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  return layout(*c).total;
}

TXL_API txl_status txl_stack_create(const txl_stack_config *c, const txl_stack_weights *w,
                                    void *persistent, size_t persistent_bytes,
                                    hipStream_t stream, txl_stack **out) {
  txl_status st = check_config(c);
  if (st != TXL_OK) return st;
  if (!w || !w->emb || !w->layers || !out || !persistent)
    return fail(TXL_ERR_INVALID_ARG, "stack_create: null weights, output or persistent buffer");
  if (!aligned16(w->emb) || !aligned16(persistent))
    return fail(TXL_ERR_UNSUPPORTED, "stack_create: emb / persistent not 16-byte aligned");
  for (int n = 0; n < c->n_layer; ++n) {
    const txl_layer_weights &l = w->layers[n];
    const void *ptrs[] = {l.wq, l.wk, l.wv, l.wo, l.wr, l.u, l.vb, l.ln1_g, l.ln1_b,
                          l.w1, l.w2, l.ln2_g, l.ln2_b};
    for (const void *p : ptrs) {
      if (!p) return fail(TXL_ERR_INVALID_ARG, "stack_create: layer %d has a null weight", n);
      if (!aligned16(p)) return fail(TXL_ERR_UNSUPPORTED, "stack_create: layer %d weight not 16-byte aligned", n);
    }
  }
  const size_t need = txl_stack_persistent_bytes(c);
  if (persistent_bytes < need)
    return fail(TXL_ERR_WORKSPACE, "stack_create: persistent buffer %zu < %zu bytes", persistent_bytes, need);
  txl_stack *s = new (std::nothrow) txl_stack;
  if (!s) return fail(TXL_ERR_INVALID_ARG, "stack_create: out of host memory");
  s->cfg = *c;
  if (s->cfg.ln_eps == 0.0f) s->cfg.ln_eps = 1e-5f;
  s->emb = w->emb;
  s->layers.assign(w->layers, w->layers + c->n_layer);
  s->persistent = persistent;
  s->r_bytes = need / c->n_layer;
  for (int n = 0; n < c->n_layer; ++n) {
    st = txl_rel_pos_table(TXL_BF16, c->M, c->L, c->d, c->n_head, c->d_h, s->layers[n].wr,
                           static_cast<char *>(persistent) + n * s->r_bytes, stream);
    if (st != TXL_OK) {
      delete s;
      return st;
    }
  }
  *out = s;
  return TXL_OK;
}

TXL_API void txl_stack_destroy(txl_stack *st) { delete st; }

TXL_API txl_status txl_segment_step(txl_stack *st, const int32_t *tokens, txl_mem *mems,
                                    void *h_out, void *workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!st || !tokens || !mems || !h_out || !workspace)
    return fail(TXL_ERR_INVALID_ARG, "segment_step: null argument");
  const txl_stack_config &c = st->cfg;
  const WsLayout ws = layout(c);
  if (ws_bytes < ws.total)
    return fail(TXL_ERR_WORKSPACE, "segment_step: workspace %zu < %zu bytes", ws_bytes, ws.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) || !aligned16(h_out))
    return fail(TXL_ERR_UNSUPPORTED, "segment_step: workspace must be 256-byte and h_out 16-byte aligned");
  for (int n = 0; n <= c.n_layer; ++n) {
    const txl_mem &m = mems[n];
    if (m.B != c.B || m.M != c.M || m.d != c.d || m.dtype != c.dtype)
      return fail(TXL_ERR_INVALID_ARG, "segment_step: ring %d shape differs from the stack", n);
    if (!m.valid || (c.M > 0 && !m.data))
      return fail(TXL_ERR_INVALID_ARG, "segment_step: ring %d has null data / valid", n);
    if (c.M > 0 && (m.head < 0 || m.head >= c.M))
      return fail(TXL_ERR_INVALID_ARG, "segment_step: ring %d head outside [0, M)", n);
    if ((c.M > 0 && !aligned16(m.data)) || (reinterpret_cast<uintptr_t>(m.valid) & 3u))
      return fail(TXL_ERR_UNSUPPORTED, "segment_step: ring %d misaligned", n);
  }

  char *base = static_cast<char *>(workspace);
  __bf16 *hc = reinterpret_cast<__bf16 *>(base + ws.hc);
  __bf16 *hn = reinterpret_cast<__bf16 *>(base + ws.hn);
  __bf16 *q = reinterpret_cast<__bf16 *>(base + ws.q);
  __bf16 *k = reinterpret_cast<__bf16 *>(base + ws.k);
  __bf16 *v = reinterpret_cast<__bf16 *>(base + ws.v);
  __bf16 *o = reinterpret_cast<__bf16 *>(base + ws.o);
  float *x = reinterpret_cast<float *>(base + ws.x);
  __bf16 *h1 = reinterpret_cast<__bf16 *>(base + ws.h1);
  __bf16 *f = reinterpret_cast<__bf16 *>(base + ws.f);
  const int HD = c.n_head * c.d_h;
  const int rows = c.B * c.L;
  const int ML = c.M + c.L;

  txl_status s = launch_embed(tokens, st->emb, hc, rows, c.d, c.vocab, stream);
  if (s != TXL_OK) return s;
  for (int n = 0; n < c.n_layer; ++n) {
    const txl_layer_weights &lw = st->layers[n];
    txl_mem &ring = mems[n];
    // Q = H W^Q
    s = launch_gemm(dense(hc, c.d, rows, HD, c.d, lw.wq, q, HD), kEpiStoreBf16, stream);
    if (s != TXL_OK) return s;
    // [K | V] = [ring; H] [W^K | W^V]
    GemmParams pkv = dense(nullptr, c.d, c.B * ML, 2 * HD, c.d, lw.wk, k, HD);
    pkv.gather = 1;
    pkv.ring = static_cast<const __bf16 *>(ring.data);
    pkv.seg = hc;
    pkv.valid = ring.valid;
    pkv.head = ring.head;
    pkv.memM = c.M;
    pkv.segL = c.L;
    pkv.w1 = static_cast<const __bf16 *>(lw.wv);
    pkv.n_split = HD;
    pkv.c1 = v;
    s = launch_gemm(pkv, kEpiStoreBf16, stream);
    if (s != TXL_OK) return s;
    // relative attention over the layer's memory (valid counts before the update)
    txl_rel_attn_args a = {};
    a.dtype = TXL_BF16;
    a.B = c.B;
    a.H = c.n_head;
    a.L = c.L;
    a.M = c.M;
    a.d_h = c.d_h;
    a.q = q;
    a.q_sb = static_cast<int64_t>(c.L) * HD;
    a.q_sh = c.d_h;
    a.q_sl = HD;
    a.k = k;
    a.v = v;
    a.kv_sb = static_cast<int64_t>(ML) * HD;
    a.kv_sh = c.d_h;
    a.kv_sl = HD;
    a.r = static_cast<char *>(st->persistent) + n * st->r_bytes;
    a.r_sh = c.d_h;
    a.r_sl = HD;
    a.u = lw.u;
    a.vb = lw.vb;
    a.mem_valid = ring.valid;
    a.scale = 0.0f;
    a.out = o;
    a.o_sb = static_cast<int64_t>(c.L) * HD;
    a.o_sh = c.d_h;
    a.o_sl = HD;
    a.lse = nullptr;
    s = txl_rel_attn_fwd(&a, stream);
    if (s != TXL_OK) return s;
    // the ring of layer n-1 takes H^(n-1) now that it has been read
    const void *hptr = hc;
    s = txl_mem_update(&ring, 1, &hptr, c.L, stream);
    if (s != TXL_OK) return s;
    // X = H + A W^O; H1 = LN1(X)
    GemmParams po = dense(o, HD, rows, c.d, HD, lw.wo, x, c.d);
    po.res = hc;
    po.ldres = c.d;
    s = launch_gemm(po, kEpiResidualF32, stream);
    if (s != TXL_OK) return s;
    s = launch_layernorm(x, lw.ln1_g, lw.ln1_b, h1, rows, c.d, c.ln_eps, stream);
    if (s != TXL_OK) return s;
    // F = GELU(H1 W1); X = H1 + F W2; H^(n) = LN2(X)
    s = launch_gemm(dense(h1, c.d, rows, c.d_ff, c.d, lw.w1, f, c.d_ff), kEpiGeluBf16, stream);
    if (s != TXL_OK) return s;
    GemmParams p2 = dense(f, c.d_ff, rows, c.d, c.d_ff, lw.w2, x, c.d);
    p2.res = h1;
    p2.ldres = c.d;
    s = launch_gemm(p2, kEpiResidualF32, stream);
    if (s != TXL_OK) return s;
    void *dst = (n + 1 == c.n_layer) ? h_out : static_cast<void *>(hn);
    s = launch_layernorm(x, lw.ln2_g, lw.ln2_b, dst, rows, c.d, c.ln_eps, stream);
    if (s != TXL_OK) return s;
    __bf16 *t = hc;
    hc = (n + 1 == c.n_layer) ? static_cast<__bf16 *>(h_out) : hn;
    hn = t;
  }
  const void *top = h_out;
  return txl_mem_update(&mems[c.n_layer], 1, &top, c.L, stream);
}

}  // extern "C"
