// Segment loss for evaluation ([P1] "Transformer-XL" notes, "Training Loop
// Sketch": the cross entropy of the current segment's tokens only).
//
// logits[v][n] = w_out[v] . h[n] are computed by the bf16 MFMA GEMM with the
// vocabulary as rows and the tokens as columns, so each lane holds one token
// and a run of vocabulary entries: the epilogue keeps, per token and
// 128-entry vocabulary tile, the maximum and the sum of exponentials, plus the
// target's logit; no logit is written to memory. A second kernel combines the
// tiles into log-sum-exp and the loss.
#include <cstdint>

#include "txl.h"
#include "txl_internal.h"

using namespace txl;

namespace {

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct LossLayout {
  size_t part_m, part_s, tgt, total;
};

LossLayout loss_layout(int32_t n_tok, int32_t vocab) {
  const size_t tiles = static_cast<size_t>(lse_row_tiles(vocab, n_tok));
  LossLayout w;
  size_t off = 0;
  w.part_m = off;
  off += align256(tiles * n_tok * sizeof(float));
  w.part_s = off;
  off += align256(tiles * n_tok * sizeof(float));
  w.tgt = off;
  off += align256(static_cast<size_t>(n_tok) * sizeof(float));
  w.total = off;
  return w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

TXL_API size_t txl_lm_loss_workspace_bytes(int32_t n_tok, int32_t vocab) {
  if (n_tok < 1 || vocab < 1) return 0;
  return loss_layout(n_tok, vocab).total;
}

TXL_API txl_status txl_lm_loss(const void *h, const void *w_out, const int32_t *targets,
                               int32_t n_tok, int32_t d, int32_t vocab, float *nll,
                               void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (n_tok < 0 || d < 1 || vocab < 1)
    return fail(TXL_ERR_INVALID_ARG, "lm_loss: n_tok >= 0, d >= 1 and vocab >= 1 required");
  if (n_tok == 0) return TXL_OK;
  if (!h || !w_out || !targets || !nll || !workspace)
    return fail(TXL_ERR_INVALID_ARG, "lm_loss: null argument");
  if (n_tok % 64 || d % 32)
    return fail(TXL_ERR_UNSUPPORTED, "lm_loss: n_tok must be a multiple of 64 and d of 32");
  if (!aligned16(h) || !aligned16(w_out) || (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(nll) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(TXL_ERR_UNSUPPORTED, "lm_loss: misaligned pointer");
  if (static_cast<int64_t>(vocab) * d >= (int64_t(1) << 31) ||
      static_cast<int64_t>(n_tok) * d >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "lm_loss: operands too large for 32-bit row indexing");
  const LossLayout ws = loss_layout(n_tok, vocab);
  if (ws_bytes < ws.total)
    return fail(TXL_ERR_WORKSPACE, "lm_loss: workspace %zu < %zu bytes", ws_bytes, ws.total);
  char *base = static_cast<char *>(workspace);
  float *part_m = reinterpret_cast<float *>(base + ws.part_m);
  float *part_s = reinterpret_cast<float *>(base + ws.part_s);
  float *tgt = reinterpret_cast<float *>(base + ws.tgt);

  GemmParams p = {};
  p.rows = vocab;
  p.N = n_tok;
  p.K = d;
  p.a = static_cast<const __bf16 *>(w_out);
  p.lda = d;
  p.w0 = static_cast<const __bf16 *>(h);
  p.n_split = n_tok;
  p.targets = targets;
  p.part_m = part_m;
  p.part_s = part_s;
  p.tgt = tgt;
  txl_status s = launch_gemm(p, kEpiLse, stream);
  if (s != TXL_OK) return s;
  return launch_lse_finish(part_m, part_s, tgt, targets, lse_row_tiles(vocab, n_tok), n_tok,
                           vocab, nll, stream);
}

}  // extern "C"
