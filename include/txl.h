/*
 * libtxl: the Transformer-XL relative-position memory attention step for
 * AMD MI355X (gfx950, CDNA4), as a C ABI.
 *
 * Pages this library implements (cited by title and section):
 *   [P1] zty624.github.io notes, "Transformer-XL"
 *   [P2] wq-win.github.io, "019 Transformer-XL"
 *   [P3] iopencloud.com, "Transformer-XL与长序列建模"
 *   [P4] robocikowo.com, "Transformer-XL"
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory on any call and keeps no pointer after the
 *     call returns (txl_stack keeps the weight pointers it is given; see there).
 *   - Every call is asynchronous on the caller's stream. TXL_OK means "all
 *     work enqueued"; device faults surface at the caller's next sync.
 *   - Every argument is checked before anything is enqueued: on an error
 *     nothing has been launched and outputs are untouched. txl_last_error()
 *     then holds a message (thread-local).
 *   - Element strides count elements, not bytes; the last dimension of every
 *     strided tensor is contiguous. Vector loads need every row start to be
 *     16-byte aligned (base pointers and strides), else TXL_ERR_UNSUPPORTED.
 *   - "bf16" means bfloat16 storage with fp32 accumulation; conversions to
 *     bf16 round to nearest even.
 *   - Keys are in logical order: key index j' in [0, M) is memory (oldest
 *     first), [M, M+L) is the current segment; key position j = j' - M.
 */
#ifndef TXL_H
#define TXL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TXL_API __attribute__((visibility("default")))
#define TXL_VERSION 1

typedef enum { TXL_F32 = 0, TXL_BF16 = 1 } txl_dtype;

typedef enum {
  TXL_OK = 0,
  TXL_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes */
  TXL_ERR_UNSUPPORTED = 2, /* valid request the library does not serve (d_h, alignment) */
  TXL_ERR_WORKSPACE = 3,   /* caller buffer too small */
  TXL_ERR_HIP = 4          /* a HIP launch failed; see txl_last_error() */
} txl_status;

/* ------------------------------------------------------------------------
 * Relative-position table R.
 * [P1] "Dimension Walkthrough": R has one row per relative distance, from
 * the farthest memory slot down to distance 0; [P4] glossary: R is a
 * sinusoidal embedding of the distance i - j, projected per head.
 *
 *   r[t, h*d_h + e] = sum_k S(M+L-1-t, k) * w_r[h*d_h + e, k]
 *   S(delta, k)     = sin(delta * f_k)        for k <  d/2
 *                     cos(delta * f_{k-d/2})  for k >= d/2,  f_k = 10000^(-2k/d)
 *
 * w_r : [H*d_h, d] (output-major, like a torch Linear weight), dtype.
 * r   : [M+L, H*d_h] row-major, dtype; as the per-head table of
 *       txl_rel_attn_fwd use r_sh = d_h, r_sl = H*d_h.
 * The sinusoid is evaluated in fp64, the projection accumulates in fp32.
 * Depends only on the weights and on (M, L): compute it once per model.
 * Errors: INVALID_ARG for null pointers, M < 0, L < 1, d odd or < 2,
 * H < 1, d_h < 1.
 * ------------------------------------------------------------------------ */
TXL_API txl_status txl_rel_pos_table(txl_dtype dtype, int32_t M, int32_t L,
                                     int32_t d, int32_t H, int32_t d_h,
                                     const void *w_r, void *r,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused relative-position attention over [memory; current segment].
 *
 * For batch row b, head h, query i in [0, L) and visible key position j:
 *   A_ij = (q_i + u_h) . k_j + (q_i + v_h) . R_{i-j}
 *        ( = q.k + q.R + u.k + v.R, the four terms of [P1] "Relative
 *          Positional Encoding"; the (q+u)/(q+v) form of [P3] section 2.2 )
 *   out_i = sum_j softmax_j(A_ij * scale) v_j        ([P1] "Dimension Walkthrough")
 * with R_{i-j} = r[h, M+L-1-(i-j)] (row t of r holds distance M+L-1-t).
 * Visible keys ([P1] "Causal Mask With Memory", allow(i, j)):
 *   memory  -valid_b <= j < 0      (slots beyond the row's valid count, e.g.
 *                                   after a document reset, are masked)
 *   current 0 <= j <= i
 * Masked keys get weight exactly 0 and are never read for V.
 * The position term is computed in-tile by index arithmetic (no
 * pad/reshape/slice, [P1] "Relative Shift Trick" replaced).
 * ------------------------------------------------------------------------ */
typedef struct {
  txl_dtype dtype;               /* q, k, v, r, u, vb and out share it     */
  int32_t B, H, L, M, d_h;       /* M >= 0 memory capacity; keys = M + L    */
  const void *q;                 /* [B, H, L, d_h]                          */
  int64_t q_sb, q_sh, q_sl;
  const void *k, *v;             /* [B, H, M+L, d_h], logical key order     */
  int64_t kv_sb, kv_sh, kv_sl;
  const void *r;                 /* [H, M+L, d_h], row t <-> distance M+L-1-t */
  int64_t r_sh, r_sl;
  const void *u, *vb;            /* [H, d_h] contiguous: content / position bias */
  const int32_t *mem_valid;      /* [B] device, each in [0, M]; NULL = all M valid */
  float scale;                   /* 0 => 1/sqrt(d_h)                        */
  void *out;                     /* [B, H, L, d_h]                          */
  int64_t o_sb, o_sh, o_sl;
  float *lse;                    /* [B, H, L] contiguous fp32, natural-log
                                    log-sum-exp of scaled visible scores; NULL = skip */
  float *out_f32;                /* [B, H, L, d_h] contiguous fp32: out before
                                    its rounding to bf16 (bf16 only, 16-byte
                                    aligned); NULL = skip. Training records it
                                    for txl_rel_attn_bwd (see there). */
} txl_rel_attn_args;

/* Shapes: d_h must be 64 (else UNSUPPORTED). B == 0 or L == 0: nothing to
 * do, TXL_OK. mem_valid values outside [0, M] are the caller's error (they
 * are clamped on the device). fp32 and bf16 are both served; bf16 runs the
 * MFMA kernel, fp32 a VALU kernel of the same semantics. */
TXL_API txl_status txl_rel_attn_fwd(const txl_rel_attn_args *a,
                                    hipStream_t stream);

/* The same attention with the visible keys of every query tile cut into
 * kv_splits contiguous ranges, each handled by its own workgroup, for short
 * segments whose query tiles alone cannot fill the GPU. Each range keeps its
 * own running max and sum and writes unnormalised results to `workspace`
 * (txl_rel_attn_split_workspace_bytes(B, H, L, kv_splits) device bytes,
 * 256-byte aligned); a second kernel combines them ([P1] "Dimension
 * Walkthrough": the softmax over all visible keys is the same after the
 * combination; only the fp32 summation order differs from txl_rel_attn_fwd).
 * kv_splits in [1, 64]; 1 is txl_rel_attn_fwd. Splits above 1 are built for
 * bf16 only (else UNSUPPORTED). Calls sharing a workspace must not overlap.
 * Errors: those of txl_rel_attn_fwd, WORKSPACE. */
TXL_API size_t txl_rel_attn_split_workspace_bytes(int32_t B, int32_t H, int32_t L,
                                                  int32_t kv_splits);
TXL_API txl_status txl_rel_attn_fwd_split(const txl_rel_attn_args *a, int32_t kv_splits,
                                          void *workspace, size_t ws_bytes,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gradients of txl_rel_attn_fwd (training).
 * The exact derivative of the attention above, by the chain rule through
 * the softmax: with p_ij the probabilities, dp_ij = dout_i . v_j,
 * D_i = dout_i . out_i and g_ij = scale * p_ij (dp_ij - D_i),
 *   dv_j = sum_i p_ij dout_i        dk_j = sum_i g_ij (q_i + u_h)
 *   dq_i = sum_j g_ij (k_j + R_{i-j})
 *   dR_t = sum_{b, i, j: row of R_{i-j} = t} g_ij (q_i + v_h)
 *   du_h = sum_{b,i,j} g_ij k_j     dvb_h = sum_{b,i,j} g_ij R_{i-j}
 * Memory keys receive dk / dv like the current ones: the stop-gradient of
 * [P1] "Why Stop Gradient" and [P2] "stop-gradient到底切断哪里" cuts the path
 * into the earlier segment that produced the memory; this segment's key and
 * value projections of the memory still receive gradient (the caller feeds
 * those rows to its W_K / W_V gradients and sends nothing further back).
 * Hidden keys (beyond a row's valid memory) get exactly zero.
 *
 * a      : the arguments of the forward call that produced out and lse
 *          (bf16 only, else UNSUPPORTED); a->out and a->lse are read, both
 *          required. When a->out_f32 is set (the forward wrote it), D_i is
 *          formed from that unrounded output instead of the bf16 out: the
 *          score gradient g_ij = p_ij (dp_ij - D_i) cancels to a small
 *          difference when the probabilities are spread evenly, so D's
 *          rounding error (2^-9 of |dout_i| |out_i|) would come back
 *          magnified in du, dvb and dR.
 * grads  : dout [B, H, L, d_h] bf16 (strided, 16-byte rows), and the fp32
 *          outputs, all contiguous: dq [B, H, L, d_h], dk and dv
 *          [B, H, M+L, d_h] (logical key order), dr [H, M+L, d_h] (row t <->
 *          distance M+L-1-t), du and dvb [H, d_h]. Every element of every
 *          output is written (B == 0 or L == 0: nothing is written).
 * workspace: txl_rel_attn_bwd_workspace_bytes(B, H, L, M) device bytes,
 *          256-byte aligned; it holds p and g for every query row (bf16,
 *          about 4 B per (query, key) pair). Calls sharing a workspace must
 *          not overlap.
 * Errors: those of txl_rel_attn_fwd, INVALID_ARG (null lse / gradient
 * pointers, misaligned outputs), WORKSPACE, UNSUPPORTED (fp32, B*H > 65535).
 * ------------------------------------------------------------------------ */
typedef struct {
  const void *dout;              /* [B, H, L, d_h] bf16: gradient at out    */
  int64_t do_sb, do_sh, do_sl;
  float *dq;                     /* [B, H, L, d_h]                          */
  float *dk, *dv;                /* [B, H, M+L, d_h]                        */
  float *dr;                     /* [H, M+L, d_h]                           */
  float *du, *dvb;               /* [H, d_h]                                */
} txl_rel_attn_grads;

TXL_API size_t txl_rel_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t L,
                                                int32_t M);
TXL_API txl_status txl_rel_attn_bwd(const txl_rel_attn_args *a,
                                    const txl_rel_attn_grads *grads,
                                    void *workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-layer FIFO memory as a ring buffer.
 * [P1] "Segment-Level Recurrence" and "Batched Tensor Contract": after the
 * step every layer's memory becomes Tail_M([mem; H]) (the last M states;
 * all of them while fewer; nothing when M = 0). [P4]: a FIFO buffer in GPU
 * memory whose oldest entries are overwritten.
 *
 * Ring layout: data[b, s, :] for slot s in [0, M). `head` (host state) is the
 * slot that holds the oldest state once the ring is full and the next slot
 * to be written; logical memory index j' in [0, M) lives in slot
 * (head + j') mod M. Row b holds valid[b] states: logical indices
 * [M - valid[b], M). A fresh stream starts with head = 0, valid = 0, and
 * data filled with finite values (e.g. zeros).
 * ------------------------------------------------------------------------ */
typedef struct {
  void *data;        /* [B, M, d] device, dtype                             */
  int32_t *valid;    /* [B] device                                          */
  int64_t head;      /* host; updated by txl_mem_update                     */
  int32_t B, M, d;
  txl_dtype dtype;
} txl_mem;

/* Append the segment to every ring: with L' = min(L, M), rows
 * h[n][b, L-L'+k, :] go to slot (head + k) mod M of ring n, then
 * head <- (head + L') mod M and valid[b] <- min(M, valid[b] + L).
 * h: host array of n_mems device pointers, each a [B, L, d] segment whose
 * row (b, l) starts at element (b*L + l) * h_row_stride (h_row_stride = 0
 * means d, i.e. contiguous; otherwise >= d, e.g. a view of a wider buffer),
 * 16-byte aligned rows. All rings in one call must share B, M, d and dtype;
 * one launch covers all. M == 0 or L == 0: nothing to do. Moves
 * 2*B*L'*d*sizeof(dtype) bytes per ring.
 * Errors: INVALID_ARG (ring fields, null h, h_row_stride < d), UNSUPPORTED
 * (misaligned rows or row strides), HIP. */
TXL_API txl_status txl_mem_update(txl_mem *mems, int32_t n_mems,
                                  const void *const *h, int64_t h_row_stride,
                                  int32_t L, hipStream_t stream);

/* Document boundary ([P1] "Batched Streams": the reset flag is per row):
 * valid[b] <- 0 in every ring for rows with reset[b] != 0 (reset: [B] uint8
 * device; NULL resets every row). The masked reading of "clear or mask":
 * the row then attends exactly as a fresh stream. */
TXL_API txl_status txl_mem_reset_rows(txl_mem *mems, int32_t n_mems,
                                      const uint8_t *reset, hipStream_t stream);

/* Copy a ring out in logical order: out[b, j', :] = data[b, (head+j') mod M, :]
 * (out: [B, M, d] contiguous device). [P1] "Segment-Level Recurrence": the
 * memories are the whole recurrent state carried from one segment to the
 * next, so a stream is checkpointed (or two memories compared) by reading
 * them out oldest first together with the valid counts; a ring restored
 * from such a copy with head = 0 continues the stream exactly. Rows'
 * invalid prefixes are copied as they are.
 * Errors: INVALID_ARG, UNSUPPORTED (misaligned), HIP. */
TXL_API txl_status txl_mem_read_logical(const txl_mem *m, void *out,
                                        hipStream_t stream);

/* One layer's attention and the append of its segment to the layer's ring,
 * in one launch ([P1] "Segment-Level Recurrence": the memory of the next
 * segment is Tail_M of this segment's memory and hidden states, taken after
 * this segment's attention has read the memory). The result is exactly that
 * of txl_rel_attn_fwd(a) followed by txl_mem_update(mem, 1, &h, a->L): out
 * and lse bit for bit, the ring's slots, valid counts and head likewise, also
 * when a->mem_valid is mem->valid (the valid counts advance only after every
 * workgroup of the attention has read them; each batch row's workgroups
 * count themselves in that row's counter in `workspace`, and the last one
 * advances the row). The attention is latency-bound and leaves HBM mostly
 * idle; the append's copy runs in its shadow.
 *
 * a         : as for txl_rel_attn_fwd.
 * mem       : one ring with mem->B == a->B and mem->M == a->M; its head is
 *             advanced on success.
 * h         : [B, L, d] contiguous device array, the ring's dtype (L = a->L).
 *             The ring's slots must not overlap the attention's inputs.
 * workspace : txl_rel_attn_mem_update_workspace_bytes(B) device bytes
 *             (256 per batch row), 256-byte aligned, zero before the first
 *             call; every call leaves them zero. Calls sharing a workspace
 *             must not overlap.
 * fp32 attention, and rings or segments of 2 GiB or more, run as the two
 * separate launches. B == 0 or L == 0: nothing to do; M == 0: the attention
 * alone.
 * Errors: those of txl_rel_attn_fwd and txl_mem_update, INVALID_ARG (ring
 * shape differs from the attention's), WORKSPACE. */
TXL_API size_t txl_rel_attn_mem_update_workspace_bytes(int32_t B);
TXL_API txl_status txl_rel_attn_fwd_mem_update(const txl_rel_attn_args *a, txl_mem *mem,
                                               const void *h, void *workspace,
                                               size_t ws_bytes, hipStream_t stream);

/* txl_rel_attn_fwd_mem_update for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launch and the same results, bit for bit, with the
 * per-row counters in a static array of the library instead of a workspace.
 * The call allocates nothing and calls no allocating routine; the caller
 * still passes every input and output.
 *
 * The array is a file-scope device array of 4096 counters 256 bytes apart
 * (1 MiB), one copy per GPU the library runs on, held until the process
 * ends; its address is looked up once per device (hipGetSymbolAddress) on
 * the first call with that device current, so the stream must belong to
 * the current device. Each call first zeroes the counters of its B rows
 * with a kernel on `stream` (graph-capturable; no memset) and the attention
 * launch leaves them zero. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or two graphs
 * replayed concurrently) race and must not be made.
 * Errors: those of txl_rel_attn_fwd_mem_update except WORKSPACE;
 * UNSUPPORTED when B > 4096; HIP when the device or the symbol cannot be
 * resolved. */
TXL_API txl_status txl_rel_attn_fwd_mem_update_noalloc(const txl_rel_attn_args *a,
                                                       txl_mem *mem, const void *h,
                                                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * One segment through an N-layer stack ([P2] "019 Transformer-XL", section 3
 * pseudo-code; [P1] "Segment-Level Recurrence" and "Training and Inference"):
 *   H^(0) = Emb[tokens]
 *   for layer n = 1..N:
 *     Q = H^(n-1) W^Q,  K, V = [SG(M^(n-1)); H^(n-1)] W^{K,V}
 *         (memory rows read from ring n-1 in logical order; invalid slots
 *          are skipped; [P1] "Relation to KV Cache": memory holds hidden
 *          states and is projected again every segment)
 *     A = txl_rel_attn_fwd(Q, K, V, R^(n), u^(n), v^(n), valid of ring n-1)
 *     ring n-1 <- Tail_M([M^(n-1); H^(n-1)])   (after it has been read)
 *     X = LN1(H^(n-1) + A W^O);  H^(n) = LN2(X + GELU(X W1) W2)
 *   ring N <- Tail_M([M^(N); H^(N)]);  h_out = H^(N)
 * The layer body after the attention (W^O, post-LayerNorm, exact-erf GELU
 * feed-forward, no biases) is not on the pages; it is this library's reading.
 * R^(n) (txl_rel_pos_table of the layer's W_R for distances M+L-1..0) is
 * built once by txl_stack_create.
 *
 * Weights (dtype bf16, device, output-major like a torch Linear weight):
 *   wq, wk, wv, wr: [H*d_h, d]   wo: [d, H*d_h]   w1: [d_ff, d]   w2: [d, d_ff]
 *   u, vb: [H, d_h]   ln1_g, ln1_b, ln2_g, ln2_b: [d]   emb: [vocab, d]
 * Shapes served: dtype bf16, d_h = 64, d and d_ff multiples of 256, H*d_h a
 * multiple of 128, d <= 4096. Token ids outside [0, vocab) embed as zeros.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_layer, d, n_head, d_h, d_ff, vocab, B, L, M;
  float ln_eps;      /* 0 => 1e-5 */
  txl_dtype dtype;
} txl_stack_config;

typedef struct {
  const void *wq, *wk, *wv, *wo, *wr, *u, *vb, *ln1_g, *ln1_b, *w1, *w2, *ln2_g, *ln2_b;
} txl_layer_weights;

typedef struct {
  const void *emb;
  const txl_layer_weights *layers;  /* n_layer entries, host array */
} txl_stack_weights;

typedef struct txl_stack txl_stack; /* opaque host object */

/* Bytes of the caller-owned persistent device buffer that holds R per layer
 * and the counters of the layers' attention + ring append launches. */
TXL_API size_t txl_stack_persistent_bytes(const txl_stack_config *c);
/* Checks the configuration, copies the weight pointer table (the weights
 * themselves must outlive the stack), builds every layer's R into
 * `persistent` on `stream` and zeroes the counters after them (steps on
 * other streams must wait for this work), and returns a host object in *out (free it with
 * txl_stack_destroy). Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE
 * (persistent_bytes too small), HIP. */
TXL_API txl_status txl_stack_create(const txl_stack_config *c, const txl_stack_weights *w,
                                    void *persistent, size_t persistent_bytes,
                                    hipStream_t stream, txl_stack **out);
/* Bytes of the caller-owned scratch device buffer txl_segment_step needs. */
TXL_API size_t txl_segment_step_workspace_bytes(const txl_stack_config *c);
/* One segment: tokens [B, L] int32 device; mems: n_layer + 1 rings (each
 * [B, M, d] of the stack's dtype; heads are advanced); h_out [B, L, d].
 * Calls with the same workspace, or on the same stack (its layers' attention
 * + ring append launches share counters in the persistent buffer), must not
 * overlap. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. Every argument
 * and shape is checked before the first launch: on INVALID_ARG, UNSUPPORTED
 * or WORKSPACE nothing has been enqueued and no head has moved. TXL_ERR_HIP
 * means a kernel launch itself failed part way: the launches before it are
 * enqueued, the rings whose update was enqueued have advanced their heads,
 * and the stream of segments cannot continue from that state (restore the
 * rings from a checkpoint, see txl_mem_read_logical). */
TXL_API txl_status txl_segment_step(txl_stack *st, const int32_t *tokens, txl_mem *mems,
                                    void *h_out, void *workspace, size_t ws_bytes,
                                    hipStream_t stream);
TXL_API void txl_stack_destroy(txl_stack *st);

/* ------------------------------------------------------------------------
 * Training: gradients of one segment with the memory as a constant.
 * [P1] "Why Stop Gradient" and "Training Loop Sketch", [P2] section
 * "stop-gradient到底切断哪里": the memory enters the segment's graph as a
 * stop-gradient input, so backpropagation ends at this segment. The memory's
 * rows still feed the segment's keys and values, hence the W^K and W^V
 * gradients, but no gradient leaves through them toward the earlier segment
 * that wrote them (there is no memory gradient output).
 *
 * txl_segment_step_train is txl_segment_step (same arguments, same rings
 * update, same h_out) that also records in `tape` what the backward reads:
 * per layer its input H, the memory and valid counts as the layer read them,
 * Q, K, V, the attention's output and log-sum-exp, the fp32 inputs of both
 * LayerNorms, H1, the feed-forward's pre-activation and GELU output; and the
 * token ids. tape: txl_segment_tape_bytes(c) device bytes, 256-byte aligned,
 * owned by the caller; its layout is private to the library.
 *
 * txl_segment_backward: given dy = d loss / d h_out ([B, L, d] fp32 device,
 * contiguous, 16-byte aligned) and the tape of the matching training step,
 * writes (overwrites, never accumulates) every parameter gradient as fp32 in
 * the layout of the weight it belongs to (txl_layer_weights above):
 *   grads->emb [vocab, d] (rows of tokens absent from the segment are 0)
 *   grads->layers[n].wq, wk, wv, wr [H*d_h, d], wo [d, H*d_h], w1 [d_ff, d],
 *     w2 [d, d_ff], u, vb [H, d_h], ln1_g, ln1_b, ln2_g, ln2_b [d]
 * all device, 16-byte aligned (emb 4-byte), host array of n_layer entries.
 * The stack's weights must be the ones the training step ran with. The
 * position table's gradient goes through R = S W_R^T to W_R (S: the fixed
 * sinusoid rows of distances M+L-1 .. 0). Products run in bf16 with fp32
 * accumulation; every reduction has a fixed order, so repeated calls give
 * identical bits.
 * workspace: txl_segment_backward_workspace_bytes(c) device bytes, 256-byte
 * aligned. Calls sharing a workspace or a tape must not overlap; the tape is
 * read only. Errors: INVALID_ARG (null pointers), WORKSPACE (tape or
 * workspace too small), UNSUPPORTED (alignment), HIP; all but HIP are
 * reported before anything is enqueued.
 * ------------------------------------------------------------------------ */
typedef struct {
  float *wq, *wk, *wv, *wo, *wr, *u, *vb, *ln1_g, *ln1_b, *w1, *w2, *ln2_g, *ln2_b;
} txl_layer_grads;

typedef struct {
  float *emb;
  const txl_layer_grads *layers;   /* n_layer entries, host array */
} txl_stack_grads;

TXL_API size_t txl_segment_tape_bytes(const txl_stack_config *c);
TXL_API txl_status txl_segment_step_train(txl_stack *st, const int32_t *tokens, txl_mem *mems,
                                          void *h_out, void *tape, size_t tape_bytes,
                                          void *workspace, size_t ws_bytes, hipStream_t stream);
TXL_API size_t txl_segment_backward_workspace_bytes(const txl_stack_config *c);
TXL_API txl_status txl_segment_backward(txl_stack *st, const void *tape, size_t tape_bytes,
                                        const float *dy, const txl_stack_grads *grads,
                                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Evaluation with projected memory ([P1] "Relation to KV Cache": the pages'
 * memory holds hidden states and re-projects them through W^K, W^V every
 * segment, where a decoder KV cache keeps the projected keys and values).
 * With fixed weights the two give the same keys and values, so for
 * evaluation each layer may keep K and V of its memory instead and project
 * only the L new rows per segment, saving 4*B*M*d*H*d_h flops per layer.
 *
 * A cache is a sliding window over a buffer of `capacity` rows per batch row:
 * rows [start, start + M) hold the layer's memory keys / values in logical
 * order (oldest first; the first M - valid[b] of them are masked and never
 * read), and the call writes the segment's projections to rows
 * [start + M, start + M + L), so the window [start, start + M + L) is the
 * layer's key sequence. Afterwards start <- start + L and
 * valid[b] <- min(M, valid[b] + L) (the memory update of the pages, with no
 * rows moved). If the advanced window would pass the end of the buffer
 * (start + M + L > capacity), the call then moves rows [start, start + M) of
 * every batch row to [0, M) and sets start = 0: once every
 * floor((capacity - M - L) / L) + 1 segments, 2*B*M*H*d_h*sizeof(dtype) bytes
 * read and written per cache.
 * ------------------------------------------------------------------------ */
typedef struct {
  void *k, *v;       /* [B, capacity, H*d_h] device, the stack's dtype */
  int32_t *valid;    /* [B] device: valid memory rows per batch row, 0..M */
  int64_t start;     /* host: first row of the window; the call advances it */
  int32_t B, capacity, hd;  /* hd = H*d_h */
  txl_dtype dtype;
} txl_kv_cache;

/* Smallest capacity a cache of this stack accepts: 2*M + L. */
TXL_API int32_t txl_kv_cache_min_capacity(const txl_stack_config *c);
/* One segment with projected memory: tokens [B, L] int32 device; caches:
 * n_layer caches (cache n-1 serves layer n), all with the stack's B, dtype,
 * hd = H*d_h, one common capacity >= txl_kv_cache_min_capacity and one
 * common start in [0, capacity - M - L]; h_out [B, L, d]. L must be a
 * multiple of 32. Uses the workspace of txl_segment_step (same size). The
 * results equal txl_segment_step's on the same stream of segments and resets
 * (the projections of each row are computed once instead of every segment,
 * in the same order). Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP; as
 * for txl_segment_step, only TXL_ERR_HIP (a failed launch) can come after
 * work was enqueued; the caches' starts have then not moved, and the stream
 * cannot continue from that state. */
TXL_API txl_status txl_segment_step_kv(txl_stack *st, const int32_t *tokens,
                                       txl_kv_cache *caches, void *h_out, void *workspace,
                                       size_t ws_bytes, hipStream_t stream);
/* Document boundary for caches (as txl_mem_reset_rows): valid[b] <- 0 in
 * every cache for rows with reset[b] != 0 (NULL resets every row). */
TXL_API txl_status txl_kv_cache_reset_rows(txl_kv_cache *caches, int32_t n_caches,
                                           const uint8_t *reset, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Evaluation ([P1] "Stream Sampler Contract", "Batched Streams", "Training
 * Loop Sketch").
 *
 * Stream sampler (host only, no device work): every batch row is a state
 * machine (doc_id, offset, reset) over its own list of documents. A step
 * hands out the next up to L tokens of the row's current document and the
 * reset flag the row held before the step; a row that reaches the end of its
 * document moves to its next document (cyclically) at offset 0 with the flag
 * raised, so that the following segment starts without context. Readings of
 * this library: a token's target is the next token of the same document (the
 * last token of a document has none); a segment shorter than L is padded to
 * L with pad_id and its padded positions have no target (-1).
 *
 * doc_tokens holds all documents back to back: document k is
 * doc_tokens[doc_offsets[k] .. doc_offsets[k+1]) (n_docs + 1 non-decreasing
 * offsets; every document non-empty). Row b streams documents
 * row_docs[row_offsets[b] .. row_offsets[b+1]) in that order (at least one per
 * row). The sampler copies what it needs; the caller's arrays may be freed
 * after the call. Every row starts at its first document with reset raised.
 * ------------------------------------------------------------------------ */
typedef struct txl_stream_sampler txl_stream_sampler; /* opaque host object */

TXL_API txl_status txl_sampler_create(int32_t B, int32_t L, const int32_t *doc_tokens,
                                      const int64_t *doc_offsets, int32_t n_docs,
                                      const int32_t *row_offsets, const int32_t *row_docs,
                                      int32_t pad_id, txl_stream_sampler **out);
/* The next segment of every row, into host arrays: tokens [B, L],
 * targets [B, L] (-1 = no target), reset [B] (1 = clear the row's memory
 * before this segment: txl_mem_reset_rows / txl_kv_cache_reset_rows), and
 * lengths [B] (tokens before the padding). Any output pointer may be NULL. */
TXL_API txl_status txl_sampler_next(txl_stream_sampler *s, int32_t *tokens, int32_t *targets,
                                    uint8_t *reset, int32_t *lengths);
TXL_API void txl_sampler_destroy(txl_stream_sampler *s);

/* Segment loss: for token n with logits z = w_out h_n (one per vocabulary
 * entry), nll[n] = log(sum_v exp(z_v)) - z_{targets[n]}, and 0 where
 * targets[n] is outside [0, vocab). The logits are never stored: each
 * vocabulary tile of the bf16 MFMA product keeps, per token, its maximum and
 * its sum of exponentials, and a second kernel combines the tiles.
 * h [n_tok, d] bf16 contiguous (e.g. the stack's h_out), w_out [vocab, d] bf16
 * contiguous (e.g. the tied embedding), targets [n_tok] int32 device,
 * nll [n_tok] fp32 device. Served: n_tok a multiple of 64, d a multiple of 32,
 * 16-byte aligned pointers. workspace: txl_lm_loss_workspace_bytes(n_tok,
 * vocab) device bytes, 256-byte aligned; calls sharing it must not overlap.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
TXL_API size_t txl_lm_loss_workspace_bytes(int32_t n_tok, int32_t vocab);
TXL_API txl_status txl_lm_loss(const void *h, const void *w_out, const int32_t *targets,
                               int32_t n_tok, int32_t d, int32_t vocab, float *nll,
                               void *workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
TXL_API const char *txl_status_str(txl_status s);
TXL_API const char *txl_last_error(void);  /* thread-local; "" if none */
TXL_API int32_t txl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TXL_H */
