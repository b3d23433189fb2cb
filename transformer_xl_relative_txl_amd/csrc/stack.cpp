// N-layer stack: one segment per call, memory rings updated in place.
//
// Order of one layer n ([P2] "019 Transformer-XL", section 3 pseudo-code):
// Q from H^(n-1), K/V from [ring n-1 in logical order; H^(n-1)], relative
// attention with ring n-1's valid counts. Ring n-1 takes H^(n-1) only after
// the K/V projection has read it and the attention has read its valid
// counts: the slots being overwritten hold the oldest keys of this very layer
// ([P2] section 2: layer n reads the states layer n-1 produced for the
// previous segment). When the states are small enough, every H^(n) is kept in
// the workspace and all N+1 rings are updated by one batched call at the end
// of the step.
#include <hip/hip_runtime.h>

#include <algorithm>
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
  void *counters;  // after the R tables: the attention + ring append's per-row counters
  size_t counter_bytes;
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
  // the attention's buffer loads address a head's keys and R rows (plus a
  // tile of margin) with 32-bit byte offsets
  if ((static_cast<int64_t>(c->M) + c->L + 96) * hd * 2 >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "stack: key rows of one head span more than 2 GiB");
  return TXL_OK;
}

// K splits of a residual product (rows x N, reduction K): split only GEMMs
// whose 64x64 tiles cannot fill the chip (fewer than 512), up to 4 splits,
// each keeping a K range of at least 256.
int residual_splits(int rows, int N, int K) {
  const int64_t tiles = static_cast<int64_t>((rows + 63) / 64) * (N / 64);
  if (tiles >= 512) return 1;
  int s = 1;
  while (s < 4 && tiles * s < 1024 && K / (2 * s) >= 256) s *= 2;
  return s;
}

// Key splits of a layer's attention. Measured on the stack's shapes: with
// fewer query-tile workgroups (128 queries each, per batch row and head) than
// CUs, two splits help (B=8 H=16 L=128 M=640: 27.1 -> 24.3 us); beyond that
// the fp32 partial results and the merge cost more than the extra workgroups
// bring (B=16 H=8 L=384 M=384: 35.8 -> 47.7 us with two), so no split.
int attn_splits(const txl_stack_config &c) {
  const int64_t grid = static_cast<int64_t>((c.L + 127) / 128) * c.B * c.n_head;
  const int tiles = (c.M + c.L + 63) / 64;
  return (grid < 256 && tiles >= 4) ? 2 : 1;
}

// Whether the ring step keeps every H^(n) and updates all rings with one
// batched call at the end (one launch instead of N+1), or updates ring n-1
// right after layer n with two alternating buffers. Measured: batching pays
// while the kept states stay small (18-layer d=1024 B*L=1024: 38 MB, step
// 2.85 -> 2.81 ms) and costs more in cache misses than it saves in launches
// when they are large (16-layer d=512 B*L=6144: 101 MB, 2.68 -> 2.75 ms).
bool batch_rings(const txl_stack_config &c) {
  const size_t bytes = static_cast<size_t>(c.n_layer) * c.B * c.L * c.d * 2;
  return bytes <= (size_t(64) << 20);
}

struct WsLayout {
  size_t hs, q, k, v, o, x, h1, f, attn, attn_bytes, total;
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
  // H^(0) .. H^(N-1) kept until the rings take them at the end of the step,
  // or two alternating slots
  w.hs = take(static_cast<size_t>(batch_rings(c) ? std::max(c.n_layer, 2) : 2) * rows * c.d * 2);
  w.q = take(rows * hd * 2);
  w.k = take(krows * hd * 2);
  w.v = take(krows * hd * 2);
  w.o = take(rows * hd * 2);
  const int HDi = c.n_head * c.d_h;
  const int rws = c.B * c.L;
  const int parts = std::max(residual_splits(rws, c.d, HDi), residual_splits(rws, c.d, c.d_ff));
  w.x = take(static_cast<size_t>(parts) * rows * c.d * 4);
  w.h1 = take(rows * c.d * 2);
  w.f = take(rows * static_cast<size_t>(c.d_ff) * 2);
  const int splits = attn_splits(c);
  w.attn_bytes = splits > 1 ? txl_rel_attn_split_workspace_bytes(c.B, c.n_head, c.L, splits) : 0;
  w.attn = take(w.attn_bytes);
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

struct StepBufs {
  __bf16 *hs, *q, *k, *v, *o, *h1, *f;
  float *x;
  void *attn;
  size_t attn_bytes;
};

StepBufs bufs(const WsLayout &ws, void *workspace) {
  char *base = static_cast<char *>(workspace);
  StepBufs b;
  b.hs = reinterpret_cast<__bf16 *>(base + ws.hs);
  b.q = reinterpret_cast<__bf16 *>(base + ws.q);
  b.k = reinterpret_cast<__bf16 *>(base + ws.k);
  b.v = reinterpret_cast<__bf16 *>(base + ws.v);
  b.o = reinterpret_cast<__bf16 *>(base + ws.o);
  b.x = reinterpret_cast<float *>(base + ws.x);
  b.h1 = reinterpret_cast<__bf16 *>(base + ws.h1);
  b.f = reinterpret_cast<__bf16 *>(base + ws.f);
  b.attn = base + ws.attn;
  b.attn_bytes = ws.attn_bytes;
  return b;
}

txl_status check_workspace(const WsLayout &ws, const void *workspace, size_t ws_bytes,
                           const void *h_out, const char *who) {
  if (ws_bytes < ws.total)
    return fail(TXL_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, ws.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) || !aligned16(h_out))
    return fail(TXL_ERR_UNSUPPORTED, "%s: workspace must be 256-byte and h_out 16-byte aligned", who);
  return TXL_OK;
}

// y = LN(res + A W) for a product p (A, W, rows, N = d, K; output p.c0 is the
// fp32 scratch x): one GEMM with the residual in its epilogue, or, when the
// tiles cannot fill the chip, a split-K GEMM writing fp32 partials that the
// LayerNorm adds up in split order before the residual.
// x_out (training) receives the fp32 sum the LayerNorm normalises.
txl_status residual_ln(GemmParams p, const __bf16 *res, const void *gamma, const void *beta,
                       void *y, float eps, hipStream_t stream, float *x_out = nullptr) {
  const int splits = residual_splits(p.rows, p.N, p.K);
  txl_status s;
  if (splits > 1) {
    p.k_splits = splits;
    p.c_split_stride = static_cast<int64_t>(p.rows) * p.ldc;
    s = launch_gemm(p, kEpiPartialF32, stream);
    if (s != TXL_OK) return s;
    return launch_layernorm(static_cast<const float *>(p.c0), splits, p.c_split_stride, res, gamma,
                            beta, y, p.rows, p.N, eps, stream, x_out);
  }
  p.res = res;
  p.ldres = p.N;
  s = launch_gemm(p, kEpiResidualF32, stream);
  if (s != TXL_OK) return s;
  return launch_layernorm(static_cast<const float *>(p.c0), 1, 0, nullptr, gamma, beta, y, p.rows,
                          p.N, eps, stream, x_out);
}

// What the training step records of layer n for the backward (all device
// pointers into the caller's tape).
struct TapeLayer {
  __bf16 *hin;   // H^(n) [B*L, d], the layer's input
  __bf16 *mem;   // ring n before the step, logical order [B, M, d]
  int32_t *valid;  // its valid counts [B]
  __bf16 *q;     // [B*L, HD]
  __bf16 *k, *v; // [B*(M+L), HD]
  __bf16 *o;     // attention output [B*L, HD]
  float *o32;    // the same before its rounding, [B, H, L, 64]
  float *lse;    // [B, H, L]
  float *x1;     // H + A W^O before LN1 [B*L, d]
  __bf16 *h1;    // LN1 output [B*L, d]
  __bf16 *fpre;  // H1 W1 before GELU [B*L, d_ff]
  __bf16 *f;     // GELU output [B*L, d_ff]
  float *x2;     // H1 + F W2 before LN2 [B*L, d]
};

struct TapeLayout {
  size_t hin, mem, valid, q, k, v, o, o32, lse, x1, h1, fpre, f, x2, per_layer, tokens, total;
};

TapeLayout tape_layout(const txl_stack_config &c) {
  const size_t hd = static_cast<size_t>(c.n_head) * c.d_h;
  const size_t rows = static_cast<size_t>(c.B) * c.L;
  const size_t krows = static_cast<size_t>(c.B) * (c.M + c.L);
  TapeLayout t;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  t.hin = take(rows * c.d * 2);
  t.mem = take(static_cast<size_t>(c.B) * c.M * c.d * 2);
  t.valid = take(static_cast<size_t>(c.B) * 4);
  t.q = take(rows * hd * 2);
  t.k = take(krows * hd * 2);
  t.v = take(krows * hd * 2);
  t.o = take(rows * hd * 2);
  t.o32 = take(rows * hd * 4);
  t.lse = take(static_cast<size_t>(c.B) * c.n_head * c.L * 4);
  t.x1 = take(rows * c.d * 4);
  t.h1 = take(rows * c.d * 2);
  t.fpre = take(rows * c.d_ff * 2);
  t.f = take(rows * c.d_ff * 2);
  t.x2 = take(rows * c.d * 4);
  t.per_layer = off;
  t.tokens = off * c.n_layer;  // after the layers: the segment's token ids
  t.total = t.tokens + align256(rows * 4);
  return t;
}

TapeLayer tape_at(const TapeLayout &t, const void *tape, int n) {
  char *base = const_cast<char *>(static_cast<const char *>(tape)) + t.per_layer * n;
  TapeLayer l;
  l.hin = reinterpret_cast<__bf16 *>(base + t.hin);
  l.mem = reinterpret_cast<__bf16 *>(base + t.mem);
  l.valid = reinterpret_cast<int32_t *>(base + t.valid);
  l.q = reinterpret_cast<__bf16 *>(base + t.q);
  l.k = reinterpret_cast<__bf16 *>(base + t.k);
  l.v = reinterpret_cast<__bf16 *>(base + t.v);
  l.o = reinterpret_cast<__bf16 *>(base + t.o);
  l.o32 = reinterpret_cast<float *>(base + t.o32);
  l.lse = reinterpret_cast<float *>(base + t.lse);
  l.x1 = reinterpret_cast<float *>(base + t.x1);
  l.h1 = reinterpret_cast<__bf16 *>(base + t.h1);
  l.fpre = reinterpret_cast<__bf16 *>(base + t.fpre);
  l.f = reinterpret_cast<__bf16 *>(base + t.f);
  l.x2 = reinterpret_cast<float *>(base + t.x2);
  return l;
}

// A layer's seven weight-gradient products, out [rows, N] fp32 = X^T Y over
// the first K rows of X [*, ldx] and Y [*, ldy] (bf16, one segment row per
// row), in the order W2, W1, W^O, W^Q, W^K, W^V, W_R. Only the shapes matter
// for sizing (null pointers).
struct LayerDw {
  DwProblem p[7];
};
LayerDw layer_dw(const txl_stack_config &c, int R, int KR, int ML, const __bf16 *dx2b, const __bf16 *f,
                 const __bf16 *dfpre, const __bf16 *h1, const __bf16 *dx1b, const __bf16 *o,
                 const __bf16 *acat, const __bf16 *hin, const __bf16 *kvg, const __bf16 *ext,
                 const __bf16 *drb, const __bf16 *st_rows, const txl_layer_grads *g) {
  const int HD = c.n_head * c.d_h;
  LayerDw L;
  L.p[0] = {dx2b, c.d, c.d, f, c.d_ff, c.d_ff, R, g ? g->w2 : nullptr};
  L.p[1] = {dfpre, c.d_ff, c.d_ff, h1, c.d, c.d, R, g ? g->w1 : nullptr};
  L.p[2] = {dx1b, c.d, c.d, o, HD, HD, R, g ? g->wo : nullptr};
  L.p[3] = {acat, 3 * HD, HD, hin, c.d, c.d, R, g ? g->wq : nullptr};
  L.p[4] = {kvg, 2 * HD, HD, ext, c.d, c.d, KR, g ? g->wk : nullptr};
  L.p[5] = {kvg ? kvg + HD : nullptr, 2 * HD, HD, ext, c.d, c.d, KR, g ? g->wv : nullptr};
  L.p[6] = {drb, HD, HD, st_rows, c.d, c.d, ML, g ? g->wr : nullptr};
  return L;
}

// Workspace of the segment backward (one layer's intermediates, reused from
// the top layer down).
struct BwdWs {
  size_t g0, g1, dx2, dx2b, dh1, dx1, dx1b, dfpre, dout, kvg, drb, attn, attn_bytes, ext, acat, wcatT,
      wT, st, pg, pb, pg1, pb1, part, part_floats, total;
};

BwdWs bwd_ws(const txl_stack_config &c) {
  const size_t hd = static_cast<size_t>(c.n_head) * c.d_h;
  const int HD = static_cast<int>(hd);
  const size_t rows = static_cast<size_t>(c.B) * c.L;
  const size_t krows = static_cast<size_t>(c.B) * (c.M + c.L);
  const size_t ml = static_cast<size_t>(c.M + c.L);
  BwdWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t rd = rows * c.d;
  w.g0 = take(rd * 4);
  w.g1 = take(rd * 4);
  w.dx2 = take(rd * 4);
  w.dx2b = take(rd * 2);
  w.dh1 = take(rd * 4);
  w.dx1 = take(rd * 4);
  w.dx1b = take(rd * 2);
  w.dfpre = take(rows * c.d_ff * 2);
  w.dout = take(rows * hd * 2);
  w.kvg = take(krows * 2 * hd * 2);
  w.drb = take(ml * hd * 2);
  w.attn_bytes = txl_rel_attn_bwd_workspace_bytes(c.B, c.n_head, c.L, c.M);
  w.attn = take(w.attn_bytes);
  w.ext = take(krows * c.d * 2);
  w.acat = take(rows * 3 * hd * 2);
  w.wcatT = take(static_cast<size_t>(c.d) * 3 * hd * 2);
  w.wT = take((2 * static_cast<size_t>(c.d) * c.d_ff + hd * c.d) * 2);
  w.st = take(ml * c.d * 2);
  int rpb;
  const size_t ln_blocks = ln_backward_blocks(static_cast<int>(rows), &rpb);
  w.pg = take(ln_blocks * c.d * 4);   // LN2's gamma / beta partials
  w.pb = take(ln_blocks * c.d * 4);
  w.pg1 = take(ln_blocks * c.d * 4);  // LN1's (summed together at the layer's end)
  w.pb1 = take(ln_blocks * c.d * 4);
  // the split-K partials of a layer's weight-gradient batch
  const LayerDw dw = layer_dw(c, static_cast<int>(rows), static_cast<int>(krows), static_cast<int>(ml),
                              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, nullptr);
  w.part_floats = dw_batch_part_floats(dw.p, 7);
  w.part = take(w.part_floats * 4);
  w.total = off;
  return w;
}

// The part of layer n that does not depend on how memory is kept: Q = H W^Q,
// relative attention over keys / values k, v ([B, M+L, H*d_h] with batch
// stride kv_sb elements, memory first) masked by `valid`, X = H + A W^O,
// H1 = LN1(X), X = H1 + GELU(H1 W1) W2, dst = LN2(X).
// With `append` set, the attention also appends hc to that ring in the same
// launch (txl_rel_attn_fwd_mem_update: the ring masked by `valid` takes the
// layer's input once the attention has read its valid counts).
txl_status layer_body(const txl_stack *st, int n, const __bf16 *hc, void *dst, const void *k,
                      const void *v, int64_t kv_sb, const int32_t *valid, const StepBufs &b,
                      hipStream_t stream, txl_mem *append = nullptr,
                      const TapeLayer *tl = nullptr) {
  const txl_stack_config &c = st->cfg;
  const txl_layer_weights &lw = st->layers[n];
  const int HD = c.n_head * c.d_h;
  const int rows = c.B * c.L;
  // with a tape, the products that the backward reads land in it
  __bf16 *q_out = tl ? tl->q : b.q;
  __bf16 *o_out = tl ? tl->o : b.o;
  __bf16 *h1_out = tl ? tl->h1 : b.h1;
  __bf16 *f_out = tl ? tl->f : b.f;
  txl_status s = launch_gemm(dense(hc, c.d, rows, HD, c.d, lw.wq, q_out, HD), kEpiStoreBf16, stream);
  if (s != TXL_OK) return s;
  txl_rel_attn_args a = {};
  a.dtype = TXL_BF16;
  a.B = c.B;
  a.H = c.n_head;
  a.L = c.L;
  a.M = c.M;
  a.d_h = c.d_h;
  a.q = q_out;
  a.q_sb = static_cast<int64_t>(c.L) * HD;
  a.q_sh = c.d_h;
  a.q_sl = HD;
  a.k = k;
  a.v = v;
  a.kv_sb = kv_sb;
  a.kv_sh = c.d_h;
  a.kv_sl = HD;
  a.r = static_cast<const char *>(st->persistent) + n * st->r_bytes;
  a.r_sh = c.d_h;
  a.r_sl = HD;
  a.u = lw.u;
  a.vb = lw.vb;
  a.mem_valid = valid;
  a.scale = 0.0f;
  a.out = o_out;
  a.o_sb = static_cast<int64_t>(c.L) * HD;
  a.o_sh = c.d_h;
  a.o_sl = HD;
  a.lse = tl ? tl->lse : nullptr;
  a.out_f32 = tl ? tl->o32 : nullptr;
  const int splits = attn_splits(c);
  if (append)
    s = txl_rel_attn_fwd_mem_update(&a, append, hc, st->counters, st->counter_bytes, stream);
  else
    s = splits > 1 ? txl_rel_attn_fwd_split(&a, splits, b.attn, b.attn_bytes, stream)
                   : txl_rel_attn_fwd(&a, stream);
  if (s != TXL_OK) return s;
  // X = H + A W^O; H1 = LN1(X)
  s = residual_ln(dense(o_out, HD, rows, c.d, HD, lw.wo, b.x, c.d), hc, lw.ln1_g, lw.ln1_b, h1_out,
                  c.ln_eps, stream, tl ? tl->x1 : nullptr);
  if (s != TXL_OK) return s;
  // F = GELU(H1 W1); X = H1 + F W2; H^(n) = LN2(X)
  GemmParams p1 = dense(h1_out, c.d, rows, c.d_ff, c.d, lw.w1, f_out, c.d_ff);
  p1.pre_out = tl ? tl->fpre : nullptr;
  s = launch_gemm(p1, kEpiGeluBf16, stream);
  if (s != TXL_OK) return s;
  return residual_ln(dense(f_out, c.d_ff, rows, c.d, c.d_ff, lw.w2, b.x, c.d), h1_out, lw.ln2_g,
                     lw.ln2_b, dst, c.ln_eps, stream, tl ? tl->x2 : nullptr);
}

}  // namespace
}  // namespace txl

using namespace txl;

extern "C" {

static size_t r_table_bytes(const txl_stack_config *c) {
  const size_t hd = static_cast<size_t>(c->n_head) * c->d_h;
  return align256(static_cast<size_t>(c->M + c->L) * hd * 2);
}

TXL_API size_t txl_stack_persistent_bytes(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  return static_cast<size_t>(c->n_layer) * r_table_bytes(c) +
         align256(txl_rel_attn_mem_update_workspace_bytes(c->B));
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
  // the attention kernels' LDS limits are raised here, so that a segment
  // step makes no HIP call but its launches
  st = rel_attn_mfma_setup();
  if (st != TXL_OK) return st;
  txl_stack *s = new (std::nothrow) txl_stack;
  if (!s) return fail(TXL_ERR_INVALID_ARG, "stack_create: out of host memory");
  s->cfg = *c;
  if (s->cfg.ln_eps == 0.0f) s->cfg.ln_eps = 1e-5f;
  s->emb = w->emb;
  s->layers.assign(w->layers, w->layers + c->n_layer);
  s->persistent = persistent;
  s->r_bytes = r_table_bytes(c);
  s->counters = static_cast<char *>(persistent) + static_cast<size_t>(c->n_layer) * s->r_bytes;
  s->counter_bytes = txl_rel_attn_mem_update_workspace_bytes(c->B);
  if (s->counter_bytes > 0) {  // zero by a kernel (no memset: a caller may capture this)
    int32_t *cnt = static_cast<int32_t *>(s->counters);
    st = launch_mem_reset(&cnt, 1, static_cast<int>(s->counter_bytes / 4), nullptr, stream);
    if (st != TXL_OK) {
      delete s;
      return st;
    }
  }
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

static txl_status segment_step(txl_stack *st, const int32_t *tokens, txl_mem *mems, void *h_out,
                               void *workspace, size_t ws_bytes, void *tape, size_t tape_bytes,
                               hipStream_t stream);

TXL_API txl_status txl_segment_step(txl_stack *st, const int32_t *tokens, txl_mem *mems,
                                    void *h_out, void *workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  return segment_step(st, tokens, mems, h_out, workspace, ws_bytes, nullptr, 0, stream);
}

TXL_API size_t txl_segment_tape_bytes(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  return tape_layout(*c).total;
}

TXL_API txl_status txl_segment_step_train(txl_stack *st, const int32_t *tokens, txl_mem *mems,
                                          void *h_out, void *tape, size_t tape_bytes,
                                          void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (!tape) return fail(TXL_ERR_INVALID_ARG, "segment_step_train: null tape");
  return segment_step(st, tokens, mems, h_out, workspace, ws_bytes, tape, tape_bytes, stream);
}

TXL_API size_t txl_segment_backward_workspace_bytes(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  return bwd_ws(*c).total;
}

// Layer n from the top down (each product C = A B^T on the stack's GEMM):
//   LN2:  dX2 = LN2'(X2, dH^(n)),  dg2, db2
//   FFN:  dW2 = dX2^T F,  dFpre = (dX2 W2) * GELU'(Fpre),  dW1 = dFpre^T H1,
//         dH1 = dX2 + dFpre W1
//   LN1:  dX1 = LN1'(X1, dH1),  dg1, db1
//   out:  dW^O = dX1^T A,  dA = dX1 W^O
//   attention backward: dQ, dK, dV over [memory; segment], dR, du, dv
//   dW^Q = dQ^T H,  dW^K = dK^T [mem; H],  dW^V = dV^T [mem; H],  dW_R = dR^T S
//   dH^(n-1) = dX1 + dQ W^Q + dK_seg W^K + dV_seg W^V   (one GEMM over [dQ|dK|dV])
// The memory rows enter dW^K and dW^V only: no gradient leaves through them.
TXL_API txl_status txl_segment_backward(txl_stack *st, const void *tape, size_t tape_bytes,
                                        const float *dy, const txl_stack_grads *grads,
                                        void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (!st || !tape || !dy || !grads || !grads->layers || !grads->emb || !workspace)
    return fail(TXL_ERR_INVALID_ARG, "segment_backward: null argument");
  const txl_stack_config &c = st->cfg;
  const TapeLayout tlay = tape_layout(c);
  if (tape_bytes < tlay.total)
    return fail(TXL_ERR_WORKSPACE, "segment_backward: tape %zu < %zu bytes", tape_bytes, tlay.total);
  const BwdWs w = bwd_ws(c);
  if (ws_bytes < w.total)
    return fail(TXL_ERR_WORKSPACE, "segment_backward: workspace %zu < %zu bytes", ws_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(tape) & 255u) || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      (reinterpret_cast<uintptr_t>(dy) & 15u))
    return fail(TXL_ERR_UNSUPPORTED,
                "segment_backward: tape and workspace must be 256-byte, dy 16-byte aligned");
  for (int n = 0; n < c.n_layer; ++n) {
    const txl_layer_grads &g = grads->layers[n];
    float *outs[] = {g.wq, g.wk, g.wv, g.wo, g.wr, g.u, g.vb, g.ln1_g, g.ln1_b, g.w1, g.w2, g.ln2_g, g.ln2_b};
    for (float *o : outs) {
      if (!o) return fail(TXL_ERR_INVALID_ARG, "segment_backward: layer %d has a null gradient", n);
      if (reinterpret_cast<uintptr_t>(o) & 15u)
        return fail(TXL_ERR_UNSUPPORTED, "segment_backward: layer %d gradient not 16-byte aligned", n);
    }
  }
  if (reinterpret_cast<uintptr_t>(grads->emb) & 3u)
    return fail(TXL_ERR_INVALID_ARG, "segment_backward: emb gradient not 4-byte aligned");

  char *base = static_cast<char *>(workspace);
  auto f32 = [&](size_t off) { return reinterpret_cast<float *>(base + off); };
  auto b16 = [&](size_t off) { return reinterpret_cast<__bf16 *>(base + off); };
  const int HD = c.n_head * c.d_h;
  const int R = c.B * c.L;
  const int KR = c.B * (c.M + c.L);
  const int ML = c.M + c.L;
  float *part = f32(w.part);
  int rpb;
  const int ln_blocks = ln_backward_blocks(R, &rpb);
  __bf16 *wcatT = b16(w.wcatT), *acat = b16(w.acat), *st_rows = b16(w.st);
  __bf16 *kvg = b16(w.kvg), *drb = b16(w.drb);
  __bf16 *ext = b16(w.ext), *wT = b16(w.wT);

  // S [M+L, d]: the sinusoid rows of distances M+L-1 .. 0, shared by every layer
  txl_status s = launch_sinusoid_rows(c.M, c.L, c.d, st_rows, stream);
  if (s != TXL_OK) return s;

  // the LayerNorm backward; its gamma / beta partials (per workgroup) are
  // summed for both LayerNorms of a layer in one launch at the layer's end
  auto ln_bwd = [&](const float *x, const void *gamma, const float *dyv, float *dx, __bf16 *dxb,
                    float *pg, float *pb) {
    return launch_ln_backward(x, gamma, dyv, dx, dxb, pg, pb, R, c.d, c.ln_eps, stream);
  };

  const float *gin = dy;
  for (int n = c.n_layer - 1; n >= 0; --n) {
    const txl_layer_weights &lw = st->layers[n];
    const txl_layer_grads &g = grads->layers[n];
    const TapeLayer tl = tape_at(tlay, tape, n);
    float *gout = f32((c.n_layer - 1 - n) % 2 ? w.g1 : w.g0);
    float *dx2 = f32(w.dx2), *dh1 = f32(w.dh1), *dx1 = f32(w.dx1);
    __bf16 *dx2b = b16(w.dx2b), *dx1b = b16(w.dx1b), *dfpre = b16(w.dfpre);
    const __bf16 *w1 = static_cast<const __bf16 *>(lw.w1), *w2 = static_cast<const __bf16 *>(lw.w2);
    const __bf16 *wo = static_cast<const __bf16 *>(lw.wo);

    // the layer's weights transposed for the input-gradient products:
    // W2^T [d_ff, d], W1^T [d, d_ff], W^O^T [HD, d], [W^Q; W^K; W^V]^T [d, 3 HD]
    __bf16 *w2T = wT, *w1T = wT + static_cast<size_t>(c.d_ff) * c.d;
    __bf16 *woT = w1T + static_cast<size_t>(c.d) * c.d_ff;
    const TransposeJob jobs[6] = {
        {w2, c.d_ff, c.d, c.d_ff, w2T, c.d, 0},
        {w1, c.d, c.d_ff, c.d, w1T, c.d_ff, 0},
        {wo, HD, c.d, HD, woT, c.d, 0},
        {lw.wq, c.d, HD, c.d, wcatT, 3 * HD, 0},
        {lw.wk, c.d, HD, c.d, wcatT, 3 * HD, HD},
        {lw.wv, c.d, HD, c.d, wcatT, 3 * HD, 2 * HD}};
    if ((s = launch_transpose_batch(jobs, 6, stream)) != TXL_OK) return s;
    // LN2
    s = ln_bwd(tl.x2, lw.ln2_g, gin, dx2, dx2b, f32(w.pg), f32(w.pb));
    if (s != TXL_OK) return s;
    // dFpre = (dX2 W2) * GELU'(Fpre)
    GemmParams pf = dense(dx2b, c.d, R, c.d_ff, c.d, w2T, dfpre, c.d_ff);
    pf.pre_in = tl.fpre;
    if ((s = launch_gemm(pf, kEpiGeluGradBf16, stream)) != TXL_OK) return s;
    // dH1 = dX2 + dFpre W1
    GemmParams ph = dense(dfpre, c.d_ff, R, c.d, c.d_ff, w1T, dh1, c.d);
    ph.res32 = dx2;
    ph.ldres = c.d;
    if ((s = launch_gemm(ph, kEpiResidualF32, stream)) != TXL_OK) return s;
    // LN1
    if ((s = ln_bwd(tl.x1, lw.ln1_g, dh1, dx1, dx1b, f32(w.pg1), f32(w.pb1))) != TXL_OK) return s;
    // dA = dX1 W^O
    if ((s = launch_gemm(dense(dx1b, c.d, R, HD, c.d, woT, b16(w.dout), HD), kEpiStoreBf16, stream)) !=
        TXL_OK)
      return s;
    // attention backward, with the forward's arguments as the tape holds them
    txl_rel_attn_args a = {};
    a.dtype = TXL_BF16;
    a.B = c.B;
    a.H = c.n_head;
    a.L = c.L;
    a.M = c.M;
    a.d_h = c.d_h;
    a.q = tl.q;
    a.q_sb = static_cast<int64_t>(c.L) * HD;
    a.q_sh = c.d_h;
    a.q_sl = HD;
    a.k = tl.k;
    a.v = tl.v;
    a.kv_sb = static_cast<int64_t>(ML) * HD;
    a.kv_sh = c.d_h;
    a.kv_sl = HD;
    a.r = static_cast<const char *>(st->persistent) + n * st->r_bytes;
    a.r_sh = c.d_h;
    a.r_sl = HD;
    a.u = lw.u;
    a.vb = lw.vb;
    a.mem_valid = tl.valid;
    a.scale = 0.0f;
    a.out = tl.o;
    a.o_sb = static_cast<int64_t>(c.L) * HD;
    a.o_sh = c.d_h;
    a.o_sl = HD;
    a.lse = tl.lse;
    a.out_f32 = tl.o32;
    // the gradients arrive as bf16 rows: dQ in acat's first HD columns, dK
    // and dV of every key in kvg ([B*(M+L), 2 HD]) and of the segment's keys
    // in acat's other columns, dR in drb [M+L, HD]
    txl_rel_attn_grads ag = {};
    ag.dout = b16(w.dout);
    ag.do_sb = static_cast<int64_t>(c.L) * HD;
    ag.do_sh = c.d_h;
    ag.do_sl = HD;
    ag.du = g.u;
    ag.dvb = g.vb;
    BwdRows rows = {};
    rows.dq = acat;
    rows.dq_ld = 3 * HD;
    rows.dk = kvg;
    rows.dv = kvg + HD;
    rows.kv_ld = 2 * HD;
    rows.dk_seg = acat + HD;
    rows.dv_seg = acat + 2 * HD;
    rows.seg_ld = 3 * HD;
    rows.dr = drb;
    rows.dr_ld = HD;
    if ((s = rel_attn_bwd_impl(&a, &ag, &rows, base + w.attn, w.attn_bytes, stream)) != TXL_OK) return s;
    // [memory; segment] rows for dW^K and dW^V (slots a row does not hold read as 0)
    if ((s = launch_gather_ext(tl.mem, tl.valid, tl.hin, c.B, c.M, c.L, c.d, ext, stream)) != TXL_OK)
      return s;
    // the layer's weight gradients in one batch (their inputs are all still
    // in place): dW2 = dX2^T F, dW1 = dFpre^T H1, dW^O = dX1^T A,
    // dW^Q = dQ^T H, dW^K = dK^T [mem; H], dW^V = dV^T [mem; H],
    // dW_R = dR^T S (R = S W_R^T for distances M+L-1 .. 0)
    {
      const LayerDw dw = layer_dw(c, R, KR, ML, dx2b, tl.f, dfpre, tl.h1, dx1b, tl.o, acat, tl.hin, kvg,
                                  ext, drb, st_rows, &g);
      if ((s = launch_dw_batch(dw.p, 7, part, w.part_floats, stream)) != TXL_OK) return s;
    }
    {
      const float *parts[4] = {f32(w.pg), f32(w.pb), f32(w.pg1), f32(w.pb1)};
      float *outs[4] = {g.ln2_g, g.ln2_b, g.ln1_g, g.ln1_b};
      if ((s = launch_reduce_cols(parts, outs, 4, ln_blocks, c.d, c.d, stream)) != TXL_OK) return s;
    }
    // dH^(n-1) = dX1 + [dQ | dK_seg | dV_seg] [W^Q; W^K; W^V]
    GemmParams pi = dense(acat, 3 * HD, R, c.d, 3 * HD, wcatT, gout, c.d);
    pi.res32 = dx1;
    pi.ldres = c.d;
    if ((s = launch_gemm(pi, kEpiResidualF32, stream)) != TXL_OK) return s;
    gin = gout;
  }
  // H^(0) = Emb[tokens]: each position's gradient goes to its token's row
  const int32_t *tok = reinterpret_cast<const int32_t *>(static_cast<const char *>(tape) + tlay.tokens);
  return launch_embed_backward(tok, R, gin, c.d, c.vocab, grads->emb, stream);
}

static txl_status segment_step(txl_stack *st, const int32_t *tokens, txl_mem *mems, void *h_out,
                               void *workspace, size_t ws_bytes, void *tape, size_t tape_bytes,
                               hipStream_t stream) {
  if (!st || !tokens || !mems || !h_out || !workspace)
    return fail(TXL_ERR_INVALID_ARG, "segment_step: null argument");
  const txl_stack_config &c = st->cfg;
  const WsLayout ws = layout(c);
  txl_status s = check_workspace(ws, workspace, ws_bytes, h_out, "segment_step");
  if (s != TXL_OK) return s;
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

  const TapeLayout tlay = tape_layout(c);
  if (tape) {
    if (tape_bytes < tlay.total)
      return fail(TXL_ERR_WORKSPACE, "segment_step_train: tape %zu < %zu bytes", tape_bytes, tlay.total);
    if (reinterpret_cast<uintptr_t>(tape) & 255u)
      return fail(TXL_ERR_UNSUPPORTED, "segment_step_train: tape not 256-byte aligned");
  }

  StepBufs b = bufs(ws, workspace);
  const int HD = c.n_head * c.d_h;
  const int rows = c.B * c.L;
  const int ML = c.M + c.L;
  // H^(n), the input of layer n, lives in slot n until the end of the step
  // (batched ring update) or in slot n mod 2 (ring updated after the layer);
  // with a tape, in the tape's record of layer n
  const bool batched = batch_rings(c);
  auto slot = [&](int n) {
    if (tape) return tape_at(tlay, tape, n).hin;
    return b.hs + static_cast<size_t>(batched ? n : (n & 1)) * rows * c.d;
  };
  s = launch_embed(tokens, st->emb, slot(0), rows, c.d, c.vocab, stream);
  if (s != TXL_OK) return s;
  if (tape) {
    s = launch_copy_i32(tokens, reinterpret_cast<int32_t *>(static_cast<char *>(tape) + tlay.tokens),
                        rows, stream);
    if (s != TXL_OK) return s;
  }
  for (int n = 0; n < c.n_layer; ++n) {
    const txl_layer_weights &lw = st->layers[n];
    txl_mem &ring = mems[n];
    const __bf16 *hc = slot(n);
    TapeLayer tl;
    if (tape) {  // the memory as this layer reads it, before any update
      tl = tape_at(tlay, tape, n);
      if (c.M > 0)
        s = launch_mem_read_logical(ring.data, tl.mem, c.B, c.M, ring.head,
                                    static_cast<int64_t>(c.d) * 2, stream, ring.valid, tl.valid);
      else
        s = launch_copy_i32(ring.valid, tl.valid, c.B, stream);
      if (s != TXL_OK) return s;
    }
    __bf16 *k_out = tape ? tl.k : b.k;
    __bf16 *v_out = tape ? tl.v : b.v;
    // [K | V] = [ring; H] [W^K | W^V], memory rows gathered in logical order
    GemmParams pkv = dense(nullptr, c.d, c.B * ML, 2 * HD, c.d, lw.wk, k_out, HD);
    pkv.gather = 1;
    pkv.ring = static_cast<const __bf16 *>(ring.data);
    pkv.seg = hc;
    pkv.valid = ring.valid;
    pkv.head = ring.head;
    pkv.memM = c.M;
    pkv.segL = c.L;
    pkv.w1 = static_cast<const __bf16 *>(lw.wv);
    pkv.n_split = HD;
    pkv.c1 = v_out;
    s = launch_gemm(pkv, kEpiStoreBf16, stream);
    if (s != TXL_OK) return s;
    void *dst = (n + 1 == c.n_layer) ? h_out : static_cast<void *>(slot(n + 1));
    // Without the batched update, ring n-1 takes H^(n-1) now that layer n has
    // read it: inside the attention's launch when it runs unsplit (the copy
    // then runs in the shadow of the latency-bound attention), else after it.
    const bool fused = !batched && attn_splits(c) == 1;
    s = layer_body(st, n, hc, dst, k_out, v_out, static_cast<int64_t>(ML) * HD, ring.valid, b,
                   stream, fused ? &ring : nullptr, tape ? &tl : nullptr);
    if (s != TXL_OK) return s;
    if (!batched && !fused) {
      const void *hptr = hc;
      s = txl_mem_update(&ring, 1, &hptr, 0, c.L, stream);
      if (s != TXL_OK) return s;
    }
  }
  if (!batched) {
    const void *top = h_out;
    return txl_mem_update(&mems[c.n_layer], 1, &top, 0, c.L, stream);
  }
  // every ring takes its H^(n) at once, now that every layer has read its
  // memory and valid counts (ring n is read only by layer n+1)
  std::vector<const void *> hp(c.n_layer + 1);
  for (int n = 0; n < c.n_layer; ++n) hp[n] = slot(n);
  hp[c.n_layer] = h_out;
  return txl_mem_update(mems, c.n_layer + 1, hp.data(), 0, c.L, stream);
}

TXL_API int32_t txl_kv_cache_min_capacity(const txl_stack_config *c) {
  if (check_config(c) != TXL_OK) return 0;
  const int64_t cap = 2 * static_cast<int64_t>(c->M) + c->L;
  return cap > 0x7fffffffLL ? 0 : static_cast<int32_t>(cap);
}

TXL_API txl_status txl_segment_step_kv(txl_stack *st, const int32_t *tokens,
                                       txl_kv_cache *caches, void *h_out, void *workspace,
                                       size_t ws_bytes, hipStream_t stream) {
  if (!st || !tokens || !caches || !h_out || !workspace)
    return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: null argument");
  const txl_stack_config &c = st->cfg;
  const WsLayout ws = layout(c);
  txl_status s = check_workspace(ws, workspace, ws_bytes, h_out, "segment_step_kv");
  if (s != TXL_OK) return s;
  const int HD = c.n_head * c.d_h;
  if (c.L % 32) return fail(TXL_ERR_UNSUPPORTED, "segment_step_kv: L must be a multiple of 32");
  const int64_t cap = caches[0].capacity;
  const int64_t start = caches[0].start;
  if (cap < 2 * static_cast<int64_t>(c.M) + c.L)
    return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: capacity %lld < 2*M + L", static_cast<long long>(cap));
  if (start < 0 || start + c.M + c.L > cap)
    return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: start %lld outside [0, capacity - M - L]",
                static_cast<long long>(start));
  if (static_cast<int64_t>(c.B) * cap * 2 * HD >= (int64_t(1) << 40))
    return fail(TXL_ERR_UNSUPPORTED, "segment_step_kv: cache too large");
  for (int n = 0; n < c.n_layer; ++n) {
    const txl_kv_cache &kc = caches[n];
    if (kc.B != c.B || kc.hd != HD || kc.dtype != c.dtype)
      return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: cache %d shape differs from the stack", n);
    if (kc.capacity != cap || kc.start != start)
      return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: caches differ in capacity or start");
    if (!kc.k || !kc.v || !kc.valid)
      return fail(TXL_ERR_INVALID_ARG, "segment_step_kv: cache %d has a null pointer", n);
    if (!aligned16(kc.k) || !aligned16(kc.v) || (reinterpret_cast<uintptr_t>(kc.valid) & 3u))
      return fail(TXL_ERR_UNSUPPORTED, "segment_step_kv: cache %d misaligned", n);
  }

  StepBufs b = bufs(ws, workspace);
  const int rows = c.B * c.L;
  __bf16 *hc = b.hs, *hn = b.hs + static_cast<size_t>(rows) * c.d;
  s = launch_embed(tokens, st->emb, hc, rows, c.d, c.vocab, stream);
  if (s != TXL_OK) return s;
  for (int n = 0; n < c.n_layer; ++n) {
    const txl_layer_weights &lw = st->layers[n];
    txl_kv_cache &kc = caches[n];
    // [K | V] of the segment rows only, into window rows [start + M, start + M + L)
    GemmParams pkv = dense(hc, c.d, rows, 2 * HD, c.d, lw.wk, kc.k, HD);
    pkv.w1 = static_cast<const __bf16 *>(lw.wv);
    pkv.n_split = HD;
    pkv.c1 = kc.v;
    pkv.c_seg = c.L;
    pkv.c_bstride = cap;
    pkv.c_row0 = start + c.M;
    s = launch_gemm(pkv, kEpiStoreBf16, stream);
    if (s != TXL_OK) return s;
    void *dst = (n + 1 == c.n_layer) ? h_out : static_cast<void *>(hn);
    const int64_t w0 = start * HD;
    s = layer_body(st, n, hc, dst, static_cast<const __bf16 *>(kc.k) + w0,
                   static_cast<const __bf16 *>(kc.v) + w0, cap * HD, kc.valid, b, stream);
    if (s != TXL_OK) return s;
    __bf16 *t = hc;
    hc = static_cast<__bf16 *>(dst);
    hn = t;
  }
  // memory update: the window slides by L, the valid counts grow
  for (int base = 0; base < c.n_layer; base += kMaxRingsPerLaunch) {
    const int n = (c.n_layer - base) < kMaxRingsPerLaunch ? (c.n_layer - base) : kMaxRingsPerLaunch;
    int32_t *valid[kMaxRingsPerLaunch];
    for (int i = 0; i < n; ++i) valid[i] = caches[base + i].valid;
    s = launch_valid_advance(valid, n, c.B, c.M, c.L, stream);
    if (s != TXL_OK) return s;
  }
  int64_t next = start + c.L;
  if (next + c.M + c.L > cap) {
    // move the memory rows back to the front of the buffer (next > M: no overlap)
    for (int base = 0; base < 2 * c.n_layer; base += kMaxRingsPerLaunch) {
      const int n = (2 * c.n_layer - base) < kMaxRingsPerLaunch ? (2 * c.n_layer - base) : kMaxRingsPerLaunch;
      KVBuffers kb;
      for (int i = 0; i < n; ++i) {
        const txl_kv_cache &kc = caches[(base + i) / 2];
        kb.p[i] = ((base + i) & 1) ? kc.v : kc.k;
      }
      s = launch_kv_compact(kb, n, c.B, c.M, cap, next, static_cast<int64_t>(HD) * 2, stream);
      if (s != TXL_OK) return s;
    }
    next = 0;
  }
  for (int n = 0; n < c.n_layer; ++n) caches[n].start = next;
  return TXL_OK;
}

TXL_API txl_status txl_kv_cache_reset_rows(txl_kv_cache *caches, int32_t n_caches,
                                           const uint8_t *reset, hipStream_t stream) {
  if (n_caches < 0 || (n_caches > 0 && !caches))
    return fail(TXL_ERR_INVALID_ARG, "kv_cache_reset_rows: null caches");
  if (n_caches == 0) return TXL_OK;
  const int B = caches[0].B;
  for (int n = 0; n < n_caches; ++n)
    if (caches[n].B != B) return fail(TXL_ERR_INVALID_ARG, "kv_cache_reset_rows: caches differ in B");
  for (int n = 0; n < n_caches; ++n)
    if (B > 0 && !caches[n].valid) return fail(TXL_ERR_INVALID_ARG, "kv_cache_reset_rows: null valid");
  if (B <= 0) return B == 0 ? TXL_OK : fail(TXL_ERR_INVALID_ARG, "kv_cache_reset_rows: B < 0");
  for (int base = 0; base < n_caches; base += kMaxRingsPerLaunch) {
    const int n = (n_caches - base) < kMaxRingsPerLaunch ? (n_caches - base) : kMaxRingsPerLaunch;
    int32_t *valid[kMaxRingsPerLaunch];
    for (int i = 0; i < n; ++i) valid[i] = caches[base + i].valid;
    txl_status s = launch_mem_reset(valid, n, B, reset, stream);
    if (s != TXL_OK) return s;
  }
  return TXL_OK;
}

}  // extern "C"
