// Host layer of libtxl: argument checks, launch dispatch, error reporting.
// Every public call validates all of its arguments before enqueuing any work,
// so an error never leaves partial results behind.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "txl.h"
#include "txl_internal.h"

namespace txl {

static thread_local char g_last_error[512] = "";

txl_status fail(txl_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

txl_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(TXL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TXL_OK;
}

static bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}
static bool stride_ok(int64_t s, size_t es) {
  return s >= 0 && ((s * static_cast<int64_t>(es)) % 16) == 0;
}
static bool dtype_ok(txl_dtype t) { return t == TXL_F32 || t == TXL_BF16; }

static void clear_error() { g_last_error[0] = '\0'; }

}  // namespace txl

using namespace txl;

extern "C" {

TXL_API const char *txl_status_str(txl_status s) {
  switch (s) {
    case TXL_OK: return "ok";
    case TXL_ERR_INVALID_ARG: return "invalid argument";
    case TXL_ERR_UNSUPPORTED: return "unsupported";
    case TXL_ERR_WORKSPACE: return "workspace too small";
    case TXL_ERR_HIP: return "hip error";
  }
  return "unknown status";
}

TXL_API const char *txl_last_error(void) { return g_last_error; }

TXL_API int32_t txl_version(void) { return TXL_VERSION; }

// ---------------------------------------------------------------------------
TXL_API txl_status txl_rel_pos_table(txl_dtype dtype, int32_t M, int32_t L,
                                     int32_t d, int32_t H, int32_t d_h,
                                     const void *w_r, void *r,
                                     hipStream_t stream) {
  clear_error();
  if (!dtype_ok(dtype)) return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: bad dtype");
  if (M < 0 || L < 1) return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: need M >= 0, L >= 1");
  if (d < 2 || (d % 2) != 0) return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: d must be even and >= 2");
  if (H < 1 || d_h < 1) return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: need H >= 1, d_h >= 1");
  if (!w_r || !r) return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: null pointer");
  if (static_cast<int64_t>(M) + L > (1 << 30))
    return fail(TXL_ERR_INVALID_ARG, "rel_pos_table: M + L too large");
  return launch_rel_pos_table(dtype, M, L, d, H * d_h, w_r, r, stream);
}

// ---------------------------------------------------------------------------
// Checks the arguments and fills p; *nothing is set to true when there is no
// work (B == 0 or L == 0).
static txl_status attn_params(const txl_rel_attn_args *a, AttnParams *out, bool *nothing) {
  *nothing = false;
  if (!a) return fail(TXL_ERR_INVALID_ARG, "rel_attn: null args");
  if (!dtype_ok(a->dtype)) return fail(TXL_ERR_INVALID_ARG, "rel_attn: bad dtype");
  if (a->B < 0 || a->H < 1 || a->L < 0 || a->M < 0)
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: need B >= 0, H >= 1, L >= 0, M >= 0");
  if (a->d_h != 64)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn: d_h = %d, only 64 is built", a->d_h);
  if (static_cast<int64_t>(a->M) + a->L > (1 << 30))
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: M + L too large");
  if (!(std::isfinite(a->scale)))
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: scale is not finite");
  if (a->B == 0 || a->L == 0) {
    *nothing = true;
    return TXL_OK;
  }
  if (!a->q || !a->k || !a->v || !a->r || !a->u || !a->vb || !a->out)
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: null tensor pointer");
  const size_t es = dtype_size(a->dtype);
  const void *ptrs[] = {a->q, a->k, a->v, a->r, a->u, a->vb, a->out};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(TXL_ERR_UNSUPPORTED, "rel_attn: tensor not 16-byte aligned");
  const int64_t strides[] = {a->q_sb, a->q_sh, a->q_sl, a->kv_sb, a->kv_sh, a->kv_sl,
                             a->r_sh, a->r_sl, a->o_sb, a->o_sh, a->o_sl};
  for (int64_t s : strides)
    if (!stride_ok(s, es))
      return fail(TXL_ERR_UNSUPPORTED,
                  "rel_attn: stride %lld is negative or not a multiple of 16 bytes",
                  static_cast<long long>(s));
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u))
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: lse not 4-byte aligned");
  if (a->out_f32 && a->dtype != TXL_BF16)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn: out_f32 is built for bf16 only");
  if (a->out_f32 && (reinterpret_cast<uintptr_t>(a->out_f32) & 15u))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn: out_f32 not 16-byte aligned");
  if (a->mem_valid && (reinterpret_cast<uintptr_t>(a->mem_valid) & 3u))
    return fail(TXL_ERR_INVALID_ARG, "rel_attn: mem_valid not 4-byte aligned");

  AttnParams p = {};
  p.q = a->q; p.k = a->k; p.v = a->v; p.r = a->r; p.u = a->u; p.vb = a->vb;
  p.out = a->out; p.lse = a->lse; p.valid = a->mem_valid;
  p.out32 = a->out_f32;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_sl = a->q_sl;
  p.kv_sb = a->kv_sb; p.kv_sh = a->kv_sh; p.kv_sl = a->kv_sl;
  p.r_sh = a->r_sh; p.r_sl = a->r_sl;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_sl = a->o_sl;
  p.B = a->B; p.H = a->H; p.L = a->L; p.M = a->M;
  p.scale = a->scale != 0.0f ? a->scale : 1.0f / std::sqrt(static_cast<float>(a->d_h));
  *out = p;
  return TXL_OK;
}

TXL_API txl_status txl_rel_attn_fwd(const txl_rel_attn_args *a,
                                    hipStream_t stream) {
  clear_error();
  AttnParams p;
  bool nothing;
  txl_status st = attn_params(a, &p, &nothing);
  if (st != TXL_OK || nothing) return st;
  if (a->dtype == TXL_BF16) return launch_rel_attn_mfma(p, stream);
  return launch_rel_attn_valu(p, a->dtype, stream);
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

TXL_API size_t txl_rel_attn_split_workspace_bytes(int32_t B, int32_t H, int32_t L,
                                                  int32_t kv_splits) {
  if (B < 0 || H < 1 || L < 0 || kv_splits < 1) return 0;
  const size_t rows = static_cast<size_t>(kv_splits) * B * H * L;
  return align256(rows * 64 * sizeof(float)) + 2 * align256(rows * sizeof(float));
}

TXL_API txl_status txl_rel_attn_fwd_split(const txl_rel_attn_args *a, int32_t kv_splits,
                                          void *workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  AttnParams p;
  bool nothing;
  txl_status st = attn_params(a, &p, &nothing);
  if (st != TXL_OK || nothing) return st;
  if (kv_splits < 1 || kv_splits > 64)
    return fail(TXL_ERR_INVALID_ARG, "rel_attn_split: kv_splits must be in [1, 64]");
  if (a->dtype != TXL_BF16 && kv_splits > 1)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_split: key splits are built for bf16 only");
  if (kv_splits == 1) return a->dtype == TXL_BF16 ? launch_rel_attn_mfma(p, stream)
                                                 : launch_rel_attn_valu(p, a->dtype, stream);
  const size_t need = txl_rel_attn_split_workspace_bytes(a->B, a->H, a->L, kv_splits);
  if (!workspace || ws_bytes < need)
    return fail(TXL_ERR_WORKSPACE, "rel_attn_split: workspace %zu < %zu bytes", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_split: workspace not 256-byte aligned");
  const size_t rows = static_cast<size_t>(kv_splits) * a->B * a->H * a->L;
  char *base = static_cast<char *>(workspace);
  p.n_split = kv_splits;
  p.part_o = reinterpret_cast<float *>(base);
  p.part_m = reinterpret_cast<float *>(base + align256(rows * 64 * sizeof(float)));
  p.part_l = reinterpret_cast<float *>(base + align256(rows * 64 * sizeof(float)) +
                                       align256(rows * sizeof(float)));
  return launch_rel_attn_mfma(p, stream);
}

static txl_status check_rings(const txl_mem *mems, int32_t n_mems, const char *who);

TXL_API size_t txl_rel_attn_mem_update_workspace_bytes(int32_t B) {
  return B > 0 ? static_cast<size_t>(B) * 256 : 0;
}

// The attention and the ring append, with the per-row counters either in
// the caller's workspace (counters != null, checked by the caller) or in the
// library's static array (counters == null: no-alloc entry point).
static txl_status attn_mem_update(const txl_rel_attn_args *a, txl_mem *mem, const void *h,
                                  void *workspace, size_t ws_bytes, bool noalloc,
                                  hipStream_t stream) {
  const char *who = noalloc ? "rel_attn_mem_update_noalloc" : "rel_attn_mem_update";
  AttnParams p;
  bool nothing;
  txl_status st = attn_params(a, &p, &nothing);
  if (st != TXL_OK) return st;
  if (!mem) return fail(TXL_ERR_INVALID_ARG, "%s: null ring", who);
  st = check_rings(mem, 1, who);
  if (st != TXL_OK) return st;
  if (mem->B != a->B || mem->M != a->M)
    return fail(TXL_ERR_INVALID_ARG, "%s: ring B, M (%d, %d) differ from the "
                "attention's (%d, %d)", who, mem->B, mem->M, a->B, a->M);
  if (nothing) return TXL_OK;  // B == 0 or L == 0: no attention and no append
  if (mem->M == 0)             // nothing to append
    return a->dtype == TXL_BF16 ? launch_rel_attn_mfma(p, stream)
                                : launch_rel_attn_valu(p, a->dtype, stream);
  if (!h) return fail(TXL_ERR_INVALID_ARG, "%s: null h", who);
  const int64_t row_bytes = static_cast<int64_t>(mem->d) * dtype_size(mem->dtype);
  if (row_bytes % 16)
    return fail(TXL_ERR_UNSUPPORTED, "%s: d * sizeof(dtype) must be a multiple of 16", who);
  if (!aligned16(h) || !aligned16(mem->data))
    return fail(TXL_ERR_UNSUPPORTED, "%s: ring or h not 16-byte aligned", who);
  const int B = mem->B, M = mem->M, L = a->L;
  if (!noalloc) {
    const size_t need = txl_rel_attn_mem_update_workspace_bytes(B);
    if (!workspace || ws_bytes < need)
      return fail(TXL_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(TXL_ERR_UNSUPPORTED, "%s: workspace not 256-byte aligned", who);
  } else if (B > kNoAllocMaxRows) {
    return fail(TXL_ERR_UNSUPPORTED, "%s: B = %d exceeds the %d batch rows of the static counters",
                who, B, kNoAllocMaxRows);
  }
  const int Lp = L < M ? L : M;
  const int64_t h_bytes = static_cast<int64_t>(B) * L * row_bytes;
  const int64_t data_bytes = static_cast<int64_t>(B) * M * row_bytes;
  const int64_t limit = (int64_t(1) << 31) - 16;
  if (a->dtype != TXL_BF16 || h_bytes >= limit || data_bytes >= limit) {
    // the two as separate launches (same results, no counters)
    st = a->dtype == TXL_BF16 ? launch_rel_attn_mfma(p, stream)
                              : launch_rel_attn_valu(p, a->dtype, stream);
    if (st != TXL_OK) return st;
    RingBatch rb;
    rb.data[0] = mem->data;
    rb.valid[0] = mem->valid;
    rb.h[0] = h;
    rb.head[0] = mem->head;
    st = launch_mem_update(rb, 1, B, M, L, row_bytes, row_bytes, stream);
  } else {
    uint32_t *done = static_cast<uint32_t *>(workspace);
    if (noalloc) {
      st = noalloc_counters(B, stream, &done);
      if (st != TXL_OK) return st;
    }
    RingAppend ra = {};
    ra.h = h;
    ra.data = mem->data;
    ra.valid = mem->valid;
    ra.done = done;
    ra.head = mem->head;
    ra.B = B;
    ra.M = M;
    ra.L = L;
    ra.Lp = Lp;
    ra.cpr = static_cast<uint32_t>(row_bytes / 16);
    ra.div_cpr = make_fastdiv(ra.cpr);
    ra.div_lp = make_fastdiv(static_cast<uint32_t>(Lp));
    ra.total = static_cast<uint32_t>(static_cast<int64_t>(B) * Lp * ra.cpr);
    ra.h_bytes = static_cast<uint32_t>(h_bytes);
    ra.data_bytes = static_cast<uint32_t>(data_bytes);
    st = launch_rel_attn_mfma_append(p, ra, stream);
  }
  if (st != TXL_OK) return st;
  mem->head = (mem->head + Lp) % M;
  return TXL_OK;
}

TXL_API txl_status txl_rel_attn_fwd_mem_update(const txl_rel_attn_args *a, txl_mem *mem,
                                               const void *h, void *workspace, size_t ws_bytes,
                                               hipStream_t stream) {
  clear_error();
  return attn_mem_update(a, mem, h, workspace, ws_bytes, false, stream);
}

TXL_API txl_status txl_rel_attn_fwd_mem_update_noalloc(const txl_rel_attn_args *a, txl_mem *mem,
                                                       const void *h, hipStream_t stream) {
  clear_error();
  return attn_mem_update(a, mem, h, nullptr, 0, true, stream);
}

// ---------------------------------------------------------------------------
// Workspace of txl_rel_attn_bwd: byte offsets of its pieces, each 256-byte aligned.
struct BwdLayout {
  size_t qv, dd, pm, gm, pu, pv, pr, total;
  int64_t ldp;
};
static BwdLayout bwd_layout(int32_t B, int32_t H, int32_t L, int32_t M) {
  BwdLayout w{};
  const size_t bhl = static_cast<size_t>(B) * H * L;
  w.ldp = static_cast<int64_t>(rel_attn_bwd_ldp(M, L));
  const size_t n_mt = (static_cast<size_t>(L) + 63) / 64;
  size_t off = 0;
  w.qv = off; off += align256(bhl * 64 * 2);
  w.dd = off; off += align256(bhl * 4);
  w.pm = off; off += align256(bhl * static_cast<size_t>(w.ldp) * 2);
  w.gm = off; off += align256(bhl * static_cast<size_t>(w.ldp) * 2);
  w.pu = off; off += align256(static_cast<size_t>(B) * H * n_mt * 64 * 4);
  w.pv = off; off += align256(static_cast<size_t>(B) * H * n_mt * 64 * 4);
  w.pr = off; off += align256(static_cast<size_t>(B) * H * (static_cast<size_t>(M) + L) * 64 * 4);
  w.total = off;
  return w;
}

TXL_API size_t txl_rel_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t M) {
  if (B < 0 || H < 1 || L < 0 || M < 0) return 0;
  return bwd_layout(B, H, L, M).total;
}

TXL_API txl_status txl_rel_attn_bwd(const txl_rel_attn_args *a, const txl_rel_attn_grads *gr,
                                    void *workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  return rel_attn_bwd_impl(a, gr, nullptr, workspace, ws_bytes, stream);
}

}  // extern "C"

txl_status txl::rel_attn_bwd_impl(const txl_rel_attn_args *a, const txl_rel_attn_grads *gr,
                                  const BwdRows *rows, void *workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  AttnParams p;
  bool nothing;
  txl_status st = attn_params(a, &p, &nothing);
  if (st != TXL_OK) return st;
  if (!gr) return fail(TXL_ERR_INVALID_ARG, "rel_attn_bwd: null gradient arguments");
  if (a->dtype != TXL_BF16)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: gradients are built for bf16 inputs only");
  if (nothing) return TXL_OK;
  if (!a->lse) return fail(TXL_ERR_INVALID_ARG, "rel_attn_bwd: the forward's lse is required");
  const BwdRows rw = rows ? *rows : BwdRows{};
  if (!gr->dout || !(gr->dq || rw.dq) || !(gr->dk || rw.dk) || !(gr->dv || rw.dv) || !(gr->dr || rw.dr) ||
      !gr->du || !gr->dvb)
    return fail(TXL_ERR_INVALID_ARG, "rel_attn_bwd: null gradient pointer");
  {
    const __bf16 *rp[] = {rw.dq, rw.dk, rw.dv, rw.dk_seg, rw.dv_seg, rw.dr};
    const int64_t rl[] = {rw.dq_ld, rw.kv_ld, rw.kv_ld, rw.seg_ld, rw.seg_ld, rw.dr_ld};
    const int64_t hd = static_cast<int64_t>(a->H) * a->d_h;
    for (int i = 0; i < 6; ++i)
      if (rp[i] && ((reinterpret_cast<uintptr_t>(rp[i]) & 7u) || rl[i] < hd || rl[i] % 4))
        return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: bf16 row output %d misaligned or rows too short", i);
  }
  if (!aligned16(gr->dout))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: dout not 16-byte aligned");
  const int64_t dstr[] = {gr->do_sb, gr->do_sh, gr->do_sl};
  for (int64_t s : dstr)
    if (!stride_ok(s, 2))
      return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: dout stride %lld is negative or not a multiple of 16 bytes",
                  static_cast<long long>(s));
  const float *outs[] = {gr->dq, gr->dk, gr->dv, gr->dr, gr->du, gr->dvb};
  for (const float *o : outs)
    if (reinterpret_cast<uintptr_t>(o) & 3u)
      return fail(TXL_ERR_INVALID_ARG, "rel_attn_bwd: gradient output not 4-byte aligned");
  if (static_cast<int64_t>(a->B) * a->H > 65535)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: B * H above 65535");
  const BwdLayout w = bwd_layout(a->B, a->H, a->L, a->M);
  if (!workspace || ws_bytes < w.total)
    return fail(TXL_ERR_WORKSPACE, "rel_attn_bwd: workspace %zu < %zu bytes", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: workspace not 256-byte aligned");
  char *base = static_cast<char *>(workspace);
  BwdParams g = {};
  g.dout = static_cast<const __bf16 *>(gr->dout);
  g.do_sb = gr->do_sb; g.do_sh = gr->do_sh; g.do_sl = gr->do_sl;
  g.lse = a->lse;
  g.out32 = a->out_f32;
  g.dq = gr->dq; g.dk = gr->dk; g.dv = gr->dv; g.dr = gr->dr; g.du = gr->du; g.dvb = gr->dvb;
  g.qv = reinterpret_cast<__bf16 *>(base + w.qv);
  g.dd = reinterpret_cast<float *>(base + w.dd);
  g.pm = reinterpret_cast<__bf16 *>(base + w.pm);
  g.gm = reinterpret_cast<__bf16 *>(base + w.gm);
  g.ldp = w.ldp;
  g.part_u = reinterpret_cast<float *>(base + w.pu);
  g.part_v = reinterpret_cast<float *>(base + w.pv);
  g.part_r = reinterpret_cast<float *>(base + w.pr);
  g.rows = rw;
  return launch_rel_attn_bwd(p, g, stream);
}

extern "C" {

// ---------------------------------------------------------------------------
static txl_status check_rings(const txl_mem *mems, int32_t n_mems, const char *who) {
  if (n_mems < 0) return fail(TXL_ERR_INVALID_ARG, "%s: n_mems < 0", who);
  if (n_mems > 0 && !mems) return fail(TXL_ERR_INVALID_ARG, "%s: null mems", who);
  for (int i = 0; i < n_mems; ++i) {
    const txl_mem &m = mems[i];
    if (!dtype_ok(m.dtype)) return fail(TXL_ERR_INVALID_ARG, "%s: ring %d bad dtype", who, i);
    if (m.B < 0 || m.M < 0 || m.d < 1)
      return fail(TXL_ERR_INVALID_ARG, "%s: ring %d needs B >= 0, M >= 0, d >= 1", who, i);
    if (m.B != mems[0].B || m.M != mems[0].M || m.d != mems[0].d || m.dtype != mems[0].dtype)
      return fail(TXL_ERR_INVALID_ARG, "%s: rings in one call must share B, M, d, dtype", who);
    if (m.B > 0 && !m.valid) return fail(TXL_ERR_INVALID_ARG, "%s: ring %d null valid", who, i);
    if (m.M > 0 && m.B > 0 && !m.data) return fail(TXL_ERR_INVALID_ARG, "%s: ring %d null data", who, i);
    if (m.M > 0 && (m.head < 0 || m.head >= m.M))
      return fail(TXL_ERR_INVALID_ARG, "%s: ring %d head %lld outside [0, M)", who, i,
                  static_cast<long long>(m.head));
    if (m.valid && (reinterpret_cast<uintptr_t>(m.valid) & 3u))
      return fail(TXL_ERR_INVALID_ARG, "%s: ring %d valid not 4-byte aligned", who, i);
  }
  return TXL_OK;
}

TXL_API txl_status txl_mem_update(txl_mem *mems, int32_t n_mems,
                                  const void *const *h, int64_t h_row_stride, int32_t L,
                                  hipStream_t stream) {
  clear_error();
  txl_status st = check_rings(mems, n_mems, "mem_update");
  if (st != TXL_OK) return st;
  if (L < 0) return fail(TXL_ERR_INVALID_ARG, "mem_update: L < 0");
  if (h_row_stride < 0) return fail(TXL_ERR_INVALID_ARG, "mem_update: h_row_stride < 0");
  if (n_mems == 0 || L == 0 || mems[0].M == 0 || mems[0].B == 0) return TXL_OK;
  if (!h) return fail(TXL_ERR_INVALID_ARG, "mem_update: null h array");
  const int64_t row_bytes = static_cast<int64_t>(mems[0].d) * dtype_size(mems[0].dtype);
  if (row_bytes % 16) return fail(TXL_ERR_UNSUPPORTED, "mem_update: d * sizeof(dtype) must be a multiple of 16");
  const int64_t stride = h_row_stride == 0 ? mems[0].d : h_row_stride;
  if (stride < mems[0].d)
    return fail(TXL_ERR_INVALID_ARG, "mem_update: h_row_stride %lld < d = %d",
                static_cast<long long>(stride), mems[0].d);
  const int64_t src_row_bytes = stride * static_cast<int64_t>(dtype_size(mems[0].dtype));
  if (src_row_bytes % 16)
    return fail(TXL_ERR_UNSUPPORTED, "mem_update: h_row_stride * sizeof(dtype) must be a multiple of 16");
  if (src_row_bytes / 16 > 0xffffffffLL)
    return fail(TXL_ERR_UNSUPPORTED, "mem_update: h_row_stride too large");
  for (int i = 0; i < n_mems; ++i) {
    if (!h[i]) return fail(TXL_ERR_INVALID_ARG, "mem_update: h[%d] is null", i);
    if (!aligned16(h[i]) || !aligned16(mems[i].data))
      return fail(TXL_ERR_UNSUPPORTED, "mem_update: ring %d or h[%d] not 16-byte aligned", i, i);
  }
  const int M = mems[0].M;
  const int Lp = L < M ? L : M;
  for (int base = 0; base < n_mems; base += kMaxRingsPerLaunch) {
    const int n = (n_mems - base) < kMaxRingsPerLaunch ? (n_mems - base) : kMaxRingsPerLaunch;
    RingBatch rb;
    for (int i = 0; i < n; ++i) {
      rb.data[i] = mems[base + i].data;
      rb.valid[i] = mems[base + i].valid;
      rb.h[i] = h[base + i];
      rb.head[i] = mems[base + i].head;
    }
    st = launch_mem_update(rb, n, mems[0].B, M, L, row_bytes, src_row_bytes, stream);
    if (st != TXL_OK) return st;
  }
  for (int i = 0; i < n_mems; ++i) mems[i].head = (mems[i].head + Lp) % M;
  return TXL_OK;
}

TXL_API txl_status txl_mem_reset_rows(txl_mem *mems, int32_t n_mems,
                                      const uint8_t *reset, hipStream_t stream) {
  clear_error();
  txl_status st = check_rings(mems, n_mems, "mem_reset_rows");
  if (st != TXL_OK) return st;
  if (n_mems == 0 || mems[0].B == 0) return TXL_OK;
  for (int base = 0; base < n_mems; base += kMaxRingsPerLaunch) {
    const int n = (n_mems - base) < kMaxRingsPerLaunch ? (n_mems - base) : kMaxRingsPerLaunch;
    int32_t *valid[kMaxRingsPerLaunch];
    for (int i = 0; i < n; ++i) valid[i] = mems[base + i].valid;
    st = launch_mem_reset(valid, n, mems[0].B, reset, stream);
    if (st != TXL_OK) return st;
  }
  return TXL_OK;
}

TXL_API txl_status txl_mem_read_logical(const txl_mem *m, void *out,
                                        hipStream_t stream) {
  clear_error();
  txl_status st = check_rings(m, m ? 1 : 0, "mem_read_logical");
  if (st != TXL_OK) return st;
  if (!m) return fail(TXL_ERR_INVALID_ARG, "mem_read_logical: null ring");
  if (m->M == 0 || m->B == 0) return TXL_OK;
  if (!out) return fail(TXL_ERR_INVALID_ARG, "mem_read_logical: null out");
  const int64_t row_bytes = static_cast<int64_t>(m->d) * dtype_size(m->dtype);
  if (row_bytes % 16) return fail(TXL_ERR_UNSUPPORTED, "mem_read_logical: d * sizeof(dtype) must be a multiple of 16");
  if (!aligned16(out) || !aligned16(m->data))
    return fail(TXL_ERR_UNSUPPORTED, "mem_read_logical: not 16-byte aligned");
  return launch_mem_read_logical(m->data, out, m->B, m->M, m->head, row_bytes, stream);
}

}  // extern "C"
