// Per-row stream sampler for evaluation (host only).
//
// [P1] "Transformer-XL" notes, "Stream Sampler Contract": each batch row is a
// state machine (doc_id, offset, reset) over its own stream of documents;
// "Batched Streams": the reset flag is per row. A step hands out the next up
// to L tokens of the row's current document; at the end of the document the
// row moves to its next document at offset 0 and raises its flag, so the
// segment after it starts without context. Segments shorter than L are
// padded; a token's target is the next token of the same document.
#include <cstdint>
#include <new>
#include <vector>

#include "txl.h"
#include "txl_internal.h"

struct txl_stream_sampler {
  int32_t B, L, pad_id;
  std::vector<int32_t> tokens;        // all documents back to back
  std::vector<int64_t> doc_begin;     // per document: first token index
  std::vector<int64_t> doc_end;       //               one past its last
  std::vector<std::vector<int32_t>> row_docs;
  struct Row {
    int32_t slot;    // index into row_docs[b]
    int64_t offset;  // within the current document
    bool reset;
  };
  std::vector<Row> rows;
};

using txl::fail;

extern "C" {

TXL_API txl_status txl_sampler_create(int32_t B, int32_t L, const int32_t *doc_tokens,
                                      const int64_t *doc_offsets, int32_t n_docs,
                                      const int32_t *row_offsets, const int32_t *row_docs,
                                      int32_t pad_id, txl_stream_sampler **out) {
  if (!out || !doc_tokens || !doc_offsets || !row_offsets || !row_docs)
    return fail(TXL_ERR_INVALID_ARG, "sampler_create: null argument");
  if (B < 1 || L < 1 || n_docs < 1)
    return fail(TXL_ERR_INVALID_ARG, "sampler_create: B, L and n_docs must be positive");
  if (doc_offsets[0] < 0) return fail(TXL_ERR_INVALID_ARG, "sampler_create: negative offset");
  for (int32_t k = 0; k < n_docs; ++k)
    if (doc_offsets[k + 1] <= doc_offsets[k])
      return fail(TXL_ERR_INVALID_ARG, "sampler_create: document %d is empty or offsets decrease", k);
  if (row_offsets[0] != 0) return fail(TXL_ERR_INVALID_ARG, "sampler_create: row_offsets[0] != 0");
  for (int32_t b = 0; b < B; ++b) {
    if (row_offsets[b + 1] <= row_offsets[b])
      return fail(TXL_ERR_INVALID_ARG, "sampler_create: row %d has no document", b);
    for (int32_t j = row_offsets[b]; j < row_offsets[b + 1]; ++j)
      if (row_docs[j] < 0 || row_docs[j] >= n_docs)
        return fail(TXL_ERR_INVALID_ARG, "sampler_create: row %d names document %d of %d", b,
                    row_docs[j], n_docs);
  }
  txl_stream_sampler *s = new (std::nothrow) txl_stream_sampler;
  if (!s) return fail(TXL_ERR_INVALID_ARG, "sampler_create: out of host memory");
  s->B = B;
  s->L = L;
  s->pad_id = pad_id;
  const int64_t base = doc_offsets[0];
  s->tokens.assign(doc_tokens + base, doc_tokens + doc_offsets[n_docs]);
  s->doc_begin.resize(n_docs);
  s->doc_end.resize(n_docs);
  for (int32_t k = 0; k < n_docs; ++k) {
    s->doc_begin[k] = doc_offsets[k] - base;
    s->doc_end[k] = doc_offsets[k + 1] - base;
  }
  s->row_docs.resize(B);
  s->rows.resize(B);
  for (int32_t b = 0; b < B; ++b) {
    s->row_docs[b].assign(row_docs + row_offsets[b], row_docs + row_offsets[b + 1]);
    s->rows[b] = {0, 0, true};
  }
  *out = s;
  return TXL_OK;
}

TXL_API txl_status txl_sampler_next(txl_stream_sampler *s, int32_t *tokens, int32_t *targets,
                                    uint8_t *reset, int32_t *lengths) {
  if (!s) return fail(TXL_ERR_INVALID_ARG, "sampler_next: null sampler");
  const int32_t L = s->L;
  for (int32_t b = 0; b < s->B; ++b) {
    txl_stream_sampler::Row &row = s->rows[b];
    const std::vector<int32_t> &docs = s->row_docs[b];
    const int32_t doc = docs[row.slot];
    const int64_t begin = s->doc_begin[doc], len = s->doc_end[doc] - begin;
    const int64_t lo = row.offset;
    const int64_t n = len - lo < L ? len - lo : L;  // tokens handed out
    for (int32_t p = 0; p < L; ++p) {
      const bool in = p < n;
      const int64_t at = begin + lo + p;
      if (tokens) tokens[static_cast<int64_t>(b) * L + p] = in ? s->tokens[at] : s->pad_id;
      if (targets)
        targets[static_cast<int64_t>(b) * L + p] = (in && lo + p + 1 < len) ? s->tokens[at + 1] : -1;
    }
    if (reset) reset[b] = row.reset ? 1 : 0;
    if (lengths) lengths[b] = static_cast<int32_t>(n);
    if (lo + n == len) {  // end of the document: next one, context cleared
      row.slot = (row.slot + 1) % static_cast<int32_t>(docs.size());
      row.offset = 0;
      row.reset = true;
    } else {
      row.offset = lo + n;
      row.reset = false;
    }
  }
  return TXL_OK;
}

TXL_API void txl_sampler_destroy(txl_stream_sampler *s) { delete s; }

}  // extern "C"
