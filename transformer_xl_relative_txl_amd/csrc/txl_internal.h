// Internal declarations shared by the host layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "txl.h"

namespace txl {

// Records a formatted message as the thread's last error and returns `s`.
txl_status fail(txl_status s, const char *fmt, ...);
// Maps the last HIP launch error (if any) to TXL_ERR_HIP with its message.
txl_status check_launch(const char *what);

inline size_t dtype_size(txl_dtype t) { return t == TXL_F32 ? 4 : 2; }

// ---- attention -----------------------------------------------------------
// Validated launch parameters (strides in elements, scale already resolved).
struct AttnParams {
  const void *q, *k, *v, *r, *u, *vb;
  void *out;
  float *lse;
  float *out32;  // optional fp32 copy of out, [B*H*L, 64] contiguous (bf16 path only)
  const int32_t *valid;
  int64_t q_sb, q_sh, q_sl, kv_sb, kv_sh, kv_sl, r_sh, r_sl, o_sb, o_sh, o_sl;
  int32_t B, H, L, M;
  float scale;
  // key-range split (bf16 only): n_split > 1 workgroups per query tile, each
  // over a contiguous range of key tiles, write unnormalised O and their
  // running max / sum (base 2) here ([n_split][B*H][L] rows), then a merge
  // kernel forms out and lse
  int32_t n_split;
  float *part_o, *part_m, *part_l;
};
// fp32 / bf16 VALU kernel (one thread per query row).
txl_status launch_rel_attn_valu(const AttnParams &p, txl_dtype dt,
                                hipStream_t s);
// bf16 MFMA kernel.
txl_status launch_rel_attn_mfma(const AttnParams &p, hipStream_t s);
// Raises the LDS limits of the bf16 attention kernels (done by their first
// launch otherwise), so that a caller can take this HIP call out of a
// sequence of launches.
txl_status rel_attn_mfma_setup();

// floor(n / d) = (umulhi(n, m) + n) >> s for 0 <= n < 2^31, d >= 1
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, static_cast<uint32_t>(m), s};
}
__device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// Sum over the 64 lanes of a wave, returned to every lane, with DPP moves
// instead of LDS permutes: pairs and quads, half-rows and rows of 16 lanes
// (each lane then holds its row's sum), then the row broadcasts that carry
// rows 0-2 into row 3; lane 63 holds the total, read out as a scalar.
template <int Ctrl, int RowMask>
__device__ inline float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl,
                                                                   RowMask, 0xF, false));
}
__device__ inline float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One ring's append (txl_mem_update of a single ring) carried out by the bf16
// attention kernel in the same launch: the 16-byte chunks of the L' = min(L, M)
// new rows are spread over the threads of the workgroups with the lighter
// query tiles, which copy after their key tiles; in each batch row the
// workgroup that finishes last (counted in the row's counter, which wraps back
// to zero) advances valid[b] after every workgroup of the row has read it.
struct RingAppend {
  const void *h;        // [B, L, d] contiguous
  void *data;           // [B, M, d]
  int32_t *valid;       // [B]
  uint32_t *done;       // per batch row a counter 256 bytes apart, zero between calls
  int64_t head;
  int32_t B, M, L, Lp;
  uint32_t cpr;         // 16-byte chunks per row
  FastDiv div_cpr, div_lp;
  uint32_t total;       // chunks to move
  int32_t copy_pos0, copy_npos;  // dealing positions of the copying workgroups
  uint32_t worker_threads;  // their threads
  uint32_t rounds;      // ceil(total / worker_threads)
  uint32_t h_bytes, data_bytes;
};
// The attention of p (n_split must be 1) and the append of ra in one launch.
txl_status launch_rel_attn_mfma_append(const AttnParams &p, const RingAppend &ra, hipStream_t s);
// Batch rows served by the static counters of the no-alloc entry point.
constexpr int kNoAllocMaxRows = 4096;
// The static counters of the current device for B batch rows (B <=
// kNoAllocMaxRows), zeroed by a kernel enqueued on s.
txl_status noalloc_counters(int B, hipStream_t s, uint32_t **out);

// gradients (bf16 inputs): p holds the forward's arguments (out = the
// forward's output); g the incoming gradient, the forward's lse, the fp32
// gradient outputs (contiguous) and the workspace pieces
// The attention gradients as bf16 rows for the stack's products (each null
// pointer: not written): column h*64 + e of row b*L + i (dq), b*(M+L) + j
// (dk, dv: every key), b*L + j - M (dk_seg, dv_seg: the segment's keys) or
// t (dr: distance row t, summed over batch rows).
struct BwdRows {
  __bf16 *dq;
  int64_t dq_ld;
  __bf16 *dk, *dv;
  int64_t kv_ld;
  __bf16 *dk_seg, *dv_seg;
  int64_t seg_ld;
  __bf16 *dr;
  int64_t dr_ld;
};
struct BwdParams {
  const __bf16 *dout;
  int64_t do_sb, do_sh, do_sl;
  const float *lse;
  const float *out32;     // the forward's unrounded out [B*H*L, 64], or null
  float *dq, *dk, *dv, *dr, *du, *dvb;
  __bf16 *qv;             // [B*H*L, 64]: q + v
  float *dd;              // [B*H*L]: dout . out
  __bf16 *pm, *gm;        // [B*H*L, ldp]: score gradients by distance and by key
  int64_t ldp;
  float *part_u, *part_v; // [B*H][ceil(L/64)][64] column sums of dq's two parts
  float *part_r;          // [B][H][M+L][64] dR of each batch row
  BwdRows rows;           // bf16 row outputs (the fp32 dq, dk, dv, dr may then be null)
};
// row length of pm / gm for M memory slots and L queries
size_t rel_attn_bwd_ldp(int M, int L);
txl_status launch_rel_attn_bwd(const AttnParams &p, const BwdParams &g, hipStream_t s);
// txl_rel_attn_bwd with the bf16 row outputs of `rows` (null: none); where a
// row output is given, the matching fp32 output of `gr` may be null
txl_status rel_attn_bwd_impl(const txl_rel_attn_args *a, const txl_rel_attn_grads *gr,
                             const BwdRows *rows, void *workspace, size_t ws_bytes, hipStream_t stream);

// ---- memory ring ---------------------------------------------------------
constexpr int kMaxRingsPerLaunch = 32;
struct RingBatch {
  void *data[kMaxRingsPerLaunch];
  int32_t *valid[kMaxRingsPerLaunch];
  const void *h[kMaxRingsPerLaunch];
  int64_t head[kMaxRingsPerLaunch];
};
// segment rows are src_row_bytes apart (>= row_bytes, a multiple of 16)
txl_status launch_mem_update(const RingBatch &rb, int n, int B, int M, int L,
                             int64_t row_bytes, int64_t src_row_bytes, hipStream_t s);
txl_status launch_mem_reset(int32_t *const *valid, int n, int B,
                            const uint8_t *reset, hipStream_t s);
txl_status launch_valid_advance(int32_t *const *valid, int n, int B, int M, int L,
                                hipStream_t s);
// projected-key/value caches: up to kMaxRingsPerLaunch buffers [B, cap, row]
struct KVBuffers {
  void *p[kMaxRingsPerLaunch];
};
txl_status launch_kv_compact(const KVBuffers &kb, int n, int B, int M, int64_t cap,
                             int64_t start, int64_t row_bytes, hipStream_t s);
// the ring's slots in logical order into out [B, M, row]; with valid_src
// set, also the B valid counts into valid_dst
txl_status launch_mem_read_logical(const void *data, void *out, int B, int M,
                                   int64_t head, int64_t row_bytes,
                                   hipStream_t s, const int32_t *valid_src = nullptr,
                                   int32_t *valid_dst = nullptr);

// ---- relative-position table ---------------------------------------------
txl_status launch_rel_pos_table(txl_dtype dt, int M, int L, int d, int HD,
                                const void *w_r, void *r, hipStream_t s);
// S [M+L, d] bf16: row t = the sinusoid of distance M+L-1-t
txl_status launch_sinusoid_rows(int M, int L, int d, void *st, hipStream_t s);

// ---- segment gradients (bwd.hip) -------------------------------------------
// bf16 transposes y[c, col0 + q] = x[q, c] for q < R, c < C (x row stride
// ldx, y row stride ldy), up to kMaxTransposes in one launch; R and C
// multiples of 64, pointers 16-byte aligned, ldx, ldy, col0 multiples of 8
struct TransposeJob {
  const void *x;
  int64_t ldx;
  int R, C;
  void *y;
  int64_t ldy;
  int col0;
};
constexpr int kMaxTransposes = 8;
txl_status launch_transpose_batch(const TransposeJob *jobs, int n, hipStream_t s);
// y [B*(M+L), d] = [memory (logical order, unheld slots zero); segment] per batch row
txl_status launch_gather_ext(const void *mem, const int32_t *valid, const void *seg, int B, int M, int L,
                             int d, void *y, hipStream_t s);
// outs[k][i] = sum over s < S of parts[k][s*stride + i] in a fixed order, for
// up to four part sets in one launch, for many parts over few columns (any
// n, 4-byte aligned)
txl_status launch_reduce_cols(const float *const *parts, float *const *outs, int n_sets, int S,
                              int64_t stride, int64_t n, hipStream_t s);
int ln_backward_blocks(int rows, int *rpb);
txl_status launch_ln_backward(const float *x, const void *gamma, const float *dy, float *dx,
                              void *dxb, float *part_g, float *part_b, int rows, int d, float eps,
                              hipStream_t s);
txl_status launch_embed_backward(const int32_t *tokens, int n_tok, const float *dh0, int d,
                                 int vocab, float *demb, hipStream_t s);
txl_status launch_copy_i32(const int32_t *src, int32_t *dst, int n, hipStream_t s);

// ---- dense layers of the stack ---------------------------------------------
// kEpiPartialF32: split-K, split s stores its fp32 partial at c0 + s*c_split_stride
// kEpiLse: C is not stored; per row tile tm and column n the tile's maximum
//          and sum of exponentials over its rows go to part_m/part_s[tm*N + n],
//          and C[targets[n]][n] to tgt[n] (rows = vocabulary, columns = tokens)
// kEpiGeluGradBf16: C = acc * GELU'(pre_in) stored bf16 (the backward of the
//          feed-forward's activation); kEpiGeluBf16 also stores the
//          pre-activation acc (bf16) to pre_out when it is set
enum { kEpiStoreBf16 = 0, kEpiGeluBf16 = 1, kEpiResidualF32 = 2, kEpiPartialF32 = 3, kEpiLse = 4,
       kEpiGeluGradBf16 = 5 };
// C[m, n] = sum_k A[m, k] W[n, k]; N split at n_split between (w0, c0) and
// (w1, c1); n_split and N are multiples of 128, K a multiple of 32.
struct GemmParams {
  int rows, N, K;
  // A rows: dense (a + m*lda), or gathered over [ring memory; segment] of
  // each batch row (rows = B*(memM+segL), both with row stride lda)
  const __bf16 *a;
  int64_t lda;
  int gather;
  const __bf16 *ring, *seg;
  const int32_t *valid;
  int64_t head;
  int memM, segL;
  const __bf16 *w0, *w1;
  int n_split;
  void *c0, *c1;
  int64_t ldc;
  // output rows: C row m is row m of c0/c1, or, when c_seg > 0 (a multiple
  // of 32), row (m / c_seg) * c_bstride + c_row0 + m % c_seg
  int c_seg;
  int64_t c_bstride, c_row0;
  const __bf16 *res;  // residual [rows, ldres] for kEpiResidualF32
  int64_t ldres;
  const float *res32; // fp32 residual [rows, ldres] instead of res (kEpiResidualF32)
  __bf16 *pre_out;    // kEpiGeluBf16: pre-activation [rows, ldc] (null = not stored)
  const __bf16 *pre_in;  // kEpiGeluGradBf16: pre-activation [rows, ldc]
  // split-K (kEpiPartialF32 only): k_splits workgroups per tile, each over a
  // contiguous range of K slabs
  int k_splits;
  int64_t c_split_stride;
  // kEpiLse only
  const int32_t *targets;
  float *part_m, *part_s, *tgt;
};
txl_status launch_gemm(const GemmParams &p, int epi, hipStream_t s);
// Weight gradients: out [rows, N] fp32 = X^T Y over the first k_rows rows of
// X [*, ldx] bf16 (rows columns used) and Y [*, ldy] bf16 (N columns used);
// rows and N multiples of 64, ldx and ldy multiples of 8, x and y 16-byte
// aligned. A batch of such products runs in one launch per tile shape: each
// product's K range is split so that the splits of the whole batch carry
// about the same number of K slabs; a split product's fp32 partials go to
// `part` and are summed into out in split order afterwards (deterministic).
struct DwProblem {
  const void *x;
  int64_t ldx;
  int rows;
  const void *y;
  int64_t ldy;
  int N;
  int k_rows;
  float *out;
};
constexpr int kMaxDwProblems = 8;
// fp32 elements of `part` that launch_dw_batch needs for these shapes
size_t dw_batch_part_floats(const DwProblem *p, int n);
txl_status launch_dw_batch(const DwProblem *p, int n, float *part, size_t part_floats, hipStream_t s);
// y = LN(x) over rows of d, x = sum of n_parts fp32 buffers (part_stride
// elements apart, added in order) plus the bf16 residual res (may be null)
// x_out (may be null) receives the summed fp32 x (the LayerNorm's input)
txl_status launch_layernorm(const float *x, int n_parts, int64_t part_stride, const void *res,
                            const void *gamma, const void *beta, void *y, int rows, int d,
                            float eps, hipStream_t s, float *x_out = nullptr);
// row tiles the kEpiLse GEMM uses for `rows` rows (its part_m/part_s height)
int lse_row_tiles(int rows, int N);
// nll[n] = log(sum_t part_s[t][n] exp(part_m[t][n] - m)) + m - tgt[n] for
// targets[n] in [0, vocab), else 0
txl_status launch_lse_finish(const float *part_m, const float *part_s, const float *tgt,
                             const int32_t *targets, int n_tiles, int N, int vocab, float *nll,
                             hipStream_t s);
txl_status launch_embed(const int32_t *tokens, const void *emb, void *out, int rows, int d,
                        int vocab, hipStream_t s);

}  // namespace txl
