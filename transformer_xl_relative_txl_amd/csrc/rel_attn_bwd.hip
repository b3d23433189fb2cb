// Gradients of the relative-position attention (bf16 inputs, fp32 gradients).
//
// The forward is the one of rel_attn_mfma.hip: for query i and visible key j'
//   a_ij = (q_i + u).k_j' + (q_i + v).R_t,  t = j' + L - 1 - i
//   p_ij = softmax_j(a_ij * scale),  out_i = sum_j p_ij v_j'
// ([P1] "Transformer-XL" notes, "Relative Positional Encoding" and
// "Dimension Walkthrough"; [P3] section 2.2 for the (q+u)/(q+v) form).
// With g_ij = scale * p_ij (dout_i.v_j' - D_i), D_i = dout_i.out_i (the
// softmax Jacobian), the chain rule gives
//   dv_j' = sum_i p_ij dout_i          dk_j' = sum_i g_ij (q_i + u)
//   dq_i  = sum_j g_ij k_j' + sum_j g_ij R_t
//   dR_t  = sum_{b,i} g_ij (q_i + v)   du = sum g_ij k_j'   dv_bias = sum g_ij R_t
// Memory keys get dk / dv like the others: the stop-gradient of [P1] "Why
// Stop Gradient" ([P2] section "stop-gradient到底切断哪里") cuts the path into
// the earlier segment that produced the memory, while this segment's
// projections of it still receive gradient.
//
// Design (first version, built for clarity of the data flow):
//  * bwd_prep: D_i, and (q+u), (q+v) rounded to bf16 once.
//  * bwd_pg: one pass per query tile that recomputes the scores exactly as
//    the forward does (same MFMA layouts, band reuse and LDS diagonal read),
//    forms p from the forward's log-sum-exp, dp = dout V^T with MFMA, and
//    g; p and g go to a workspace as bf16 rows [b, h, i, j'] (staged through
//    LDS so each row segment is written by consecutive lanes).
//  * bgemm: one small MFMA kernel for the five contractions over p and g,
//    reading the visible part of each row only (hidden entries are masked on
//    load, so nothing outside the visited tiles needs clearing). The
//    position terms read g along diagonals: the element of distance row t
//    for query i is g[i][t + i - (L-1)], a matrix whose row stride is one
//    more than g's, so dq's position part and dR are ordinary products over
//    that skewed view.
//  * bwd_reduce: dR summed over batch rows (its product runs per row, for
//    parallelism), du and dv_bias from per-tile column sums of dq's two parts.
#include <hip/hip_runtime.h>

#include <cmath>

#include "txl_internal.h"

namespace txl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int DH = 64;
constexpr int QW = 32;         // queries per wave
constexpr int NW = 4;          // waves per workgroup
constexpr int BQ = QW * NW;
constexpr int BK = 64;         // keys per tile
constexpr int KS = DH + 8;     // K / V tile row stride (bf16)
constexpr int NU = 2 * QW;
constexpr int US = QW + 2;     // band row stride (floats)
constexpr int PS = BK + 4;     // p / g staging row stride (bf16): 8-byte aligned rows

constexpr size_t kLdsT = size_t(BK) * KS * 2;   // one K or V tile
constexpr size_t kLdsBand = size_t(NW) * NU * US * 4;
constexpr size_t kLdsTotal = 4 * kLdsT + kLdsBand;  // K and V, double-buffered
static_assert(size_t(2) * QW * PS * 2 <= size_t(NU) * US * 4, "p/g staging must fit a wave's band");

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ inline bf16x8 load8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<__bf16>(0.0f);
  return z;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ inline u32x4 bload(rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

// ---------------------------------------------------------------------------
// D_i = dout_i . out_i (fp32), qu = bf16(q + u), qv = bf16(q + v); one thread
// per query row and 8 dimensions.
__global__ __launch_bounds__(256) void bwd_prep_kernel(AttnParams p, BwdParams g) {
  const int64_t BHL = static_cast<int64_t>(p.B) * p.H * p.L;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = e >> 3;
  const int c = static_cast<int>(e & 7);
  float acc = 0.0f;
  if (row < BHL) {
    const int64_t bh = row / p.L;
    const int i = static_cast<int>(row - bh * p.L);
    const int b = static_cast<int>(bh / p.H), h = static_cast<int>(bh - static_cast<int64_t>(b) * p.H);
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh + i * p.q_sl + 8 * c;
    const __bf16 *op = static_cast<const __bf16 *>(p.out) + b * p.o_sb + h * p.o_sh + i * p.o_sl + 8 * c;
    const __bf16 *dp = g.dout + b * g.do_sb + h * g.do_sh + i * g.do_sl + 8 * c;
    const bf16x8 qv = load8(qp), ov = load8(op), dv = load8(dp);
    const bf16x8 uv = load8(static_cast<const __bf16 *>(p.u) + h * DH + 8 * c);
    const bf16x8 vv = load8(static_cast<const __bf16 *>(p.vb) + h * DH + 8 * c);
    bf16x8 a, bq;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float qf = static_cast<float>(qv[x]);
      a[x] = static_cast<__bf16>(qf + static_cast<float>(uv[x]));
      bq[x] = static_cast<__bf16>(qf + static_cast<float>(vv[x]));
      acc += static_cast<float>(dv[x]) * static_cast<float>(ov[x]);
    }
    *reinterpret_cast<bf16x8 *>(g.qu + row * DH + 8 * c) = a;
    *reinterpret_cast<bf16x8 *>(g.qv + row * DH + 8 * c) = bq;
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < BHL && c == 0) g.dd[row] = acc;
}

// ---------------------------------------------------------------------------
// p and g for every visited (query, key) pair of a query tile.
struct KVRegs {
  u32x4 k[2], v[2];
};
__device__ inline void load_kv(KVRegs &x, rsrc_t krs, rsrc_t vrs, int row_bytes, int j0, int tid) {
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int cidx = tid + rep * 256;
    const int off = (j0 + (cidx >> 3)) * row_bytes + (cidx & 7) * 16;
    x.k[rep] = bload(krs, off);
    x.v[rep] = bload(vrs, off);
  }
}
__device__ inline void store_kv(const KVRegs &x, __bf16 *sk, __bf16 *sv, int tid) {
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int cidx = tid + rep * 256;
    const int o = (cidx >> 3) * KS + (cidx & 7) * 8;
    *reinterpret_cast<u32x4 *>(sk + o) = x.k[rep];
    *reinterpret_cast<u32x4 *>(sv + o) = x.v[rep];
  }
}

__global__ __launch_bounds__(256, 2) void bwd_pg_kernel(AttnParams p, BwdParams g, int n_qt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float *sband = reinterpret_cast<float *>(smem + 4 * kLdsT);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.H;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.x) / BH;
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int L = p.L, M = p.M, ML = M + L;
  const int i0 = qt * BQ;
  const int iw = i0 + wave * QW;
  const int i = iw + r;

  int valid = p.valid ? p.valid[b] : M;
  valid = valid < 0 ? 0 : (valid > M ? M : valid);
  const int j_lo = M - valid;
  const int i_last = (i0 + BQ < L ? i0 + BQ : L) - 1;
  const int j_end = M + i_last + 1;
  const int n_tiles = (j_end - j_lo + BK - 1) / BK;

  const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16 *kp = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *vp = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *rp = static_cast<const __bf16 *>(p.r) + h * p.r_sh;
  const __bf16 *up = static_cast<const __bf16 *>(p.u) + h * DH;
  const __bf16 *vbp = static_cast<const __bf16 *>(p.vb) + h * DH;
  const __bf16 *dop = g.dout + b * g.do_sb + h * g.do_sh;

  const int kv_row_bytes = static_cast<int>(p.kv_sl) * 2;
  const int r_row_bytes = static_cast<int>(p.r_sl) * 2;
  const rsrc_t krs = make_rsrc(kp, static_cast<uint32_t>((j_end - 1) * kv_row_bytes + 2 * DH));
  const rsrc_t vrs = make_rsrc(vp, static_cast<uint32_t>((j_end - 1) * kv_row_bytes + 2 * DH));
  const rsrc_t rrs = make_rsrc(rp, static_cast<uint32_t>((ML - 1) * r_row_bytes + 2 * DH));

  KVRegs nxt;
  load_kv(nxt, krs, vrs, kv_row_bytes, j_lo, tid);

  // the forward's scaled operands, and dout as the B operand of dp^T = V dout^T
  const float c2 = p.scale * 1.4426950408889634f;
  bf16x8 qa[4], qb[4], dob[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int d0 = 16 * s + 8 * hh;
    const bf16x8 qv = i < L ? load8(qp + static_cast<int64_t>(i) * p.q_sl + d0) : zero8();
    dob[s] = i < L ? load8(dop + static_cast<int64_t>(i) * g.do_sl + d0) : zero8();
    const bf16x8 uv = load8(up + d0);
    const bf16x8 vv = load8(vbp + d0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = static_cast<float>(qv[e]);
      qa[s][e] = static_cast<__bf16>((x + static_cast<float>(uv[e])) * c2);
      qb[s][e] = static_cast<__bf16>((x + static_cast<float>(vv[e])) * c2);
    }
  }
  const int64_t row_bh = static_cast<int64_t>(bh) * L;
  const float lse2 = i < L ? g.lse[row_bh + i] * 1.4426950408889634f : 0.0f;
  const float dd = i < L ? g.dd[row_bh + i] : 0.0f;

  float *band = sband + wave * (NU * US);
  float *band_w = band + 4 * hh * US + r;
  const float *band_r = band + (31 - r + 4 * hh) * US + r;
  __bf16 *stg = reinterpret_cast<__bf16 *>(band);   // p rows [32][PS], then g rows

  bf16x8 rr[2][4];
  auto load_r = [&](int j0) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int off = (j0 + 32 * (bb + 1) + r + L - 32 - iw) * r_row_bytes + 16 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) rr[bb][s] = __builtin_bit_cast(bf16x8, bload(rrs, off + 32 * s));
    }
  };
  f32x16 b_carry;
  {
    bf16x8 r0[4];
    const int off = (j_lo + r + L - 32 - iw) * r_row_bytes + 16 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) r0[s] = __builtin_bit_cast(bf16x8, bload(rrs, off + 32 * s));
#pragma unroll
    for (int x = 0; x < 16; ++x) b_carry[x] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) b_carry = mfma32(r0[s], qb[s], b_carry);
  }
  load_r(j_lo);

  store_kv(nxt, reinterpret_cast<__bf16 *>(smem), reinterpret_cast<__bf16 *>(smem + kLdsT), tid);
  load_kv(nxt, krs, vrs, kv_row_bytes, j_lo + BK, tid);
  __syncthreads();

  __bf16 *pm = g.pm + row_bh * g.ldp;
  __bf16 *gm = g.gm + row_bh * g.ldp;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int j0 = j_lo + kt * BK;
    unsigned char *buf = smem + (kt & 1) * (2 * kLdsT);
    const __bf16 *sk = reinterpret_cast<const __bf16 *>(buf);
    const __bf16 *svr = reinterpret_cast<const __bf16 *>(buf + kLdsT);

    // ---- scores, exactly as the forward computes them ----
    f32x16 s_acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) s_acc[kb][x] = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        s_acc[kb] = mfma32(load8(sk + (kb * 32 + r) * KS + 16 * s + 8 * hh), qa[s], s_acc[kb]);
    }
    f32x16 b_acc[3];
    b_acc[0] = b_carry;
#pragma unroll
    for (int bb = 1; bb < 3; ++bb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) b_acc[bb][x] = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) b_acc[bb] = mfma32(rr[bb - 1][s], qb[s], b_acc[bb]);
    }
    b_carry = b_acc[2];
    load_r(j0 + BK);

    float sv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            band_w[(32 * half + 8 * a4 + cc) * US] = b_acc[kb + half][4 * a4 + cc];
      wave_lds_sync();
#pragma unroll
      for (int x = 0; x < 16; ++x) sv[kb][x] = s_acc[kb][x] + band_r[(8 * (x >> 2) + (x & 3)) * US];
      wave_lds_sync();
    }
    if (j0 + BK - 1 - M > iw) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int jj = j0 + kb * 32 + 8 * (x >> 2) + 4 * hh + (x & 3);
          if (jj - M > i) sv[kb][x] = -INFINITY;
        }
    }

    // ---- dp^T[key][query] = V dout^T ----
    f32x16 dp_acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) dp_acc[kb][x] = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dp_acc[kb] = mfma32(load8(svr + (kb * 32 + r) * KS + 16 * s + 8 * hh), dob[s], dp_acc[kb]);
    }

    // ---- p = 2^(s - lse2), g = scale p (dp - D); staged as rows [query][key] ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 p4, g4;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int x = 4 * a4 + cc;
          const float pv = __builtin_amdgcn_exp2f(sv[kb][x] - lse2);
          p4[cc] = static_cast<__bf16>(pv);
          g4[cc] = static_cast<__bf16>(p.scale * pv * (dp_acc[kb][x] - dd));
        }
        const int key = kb * 32 + 8 * a4 + 4 * hh;
        *reinterpret_cast<bf16x4 *>(stg + r * PS + key) = p4;
        *reinterpret_cast<bf16x4 *>(stg + (QW + r) * PS + key) = g4;
      }
    wave_lds_sync();
    if ((j_lo & 3) == 0) {
      // tiles start 4-aligned: 4 keys per lane, 16 lanes per row, 4 rows per store
      const int kk = (lane & 15) * 4, jj = j0 + kk;
      if (jj < ML) {
#pragma unroll
        for (int it = 0; it < QW / 4; ++it) {
          const int qq = (lane >> 4) + 4 * it, row = iw + qq;
          if (row < L) {
            *reinterpret_cast<bf16x4 *>(pm + static_cast<int64_t>(row) * g.ldp + jj) =
                *reinterpret_cast<const bf16x4 *>(stg + qq * PS + kk);
            *reinterpret_cast<bf16x4 *>(gm + static_cast<int64_t>(row) * g.ldp + jj) =
                *reinterpret_cast<const bf16x4 *>(stg + (QW + qq) * PS + kk);
          }
        }
      }
    } else {
      const int jj = j0 + lane;
      if (jj < ML) {
#pragma unroll 4
        for (int qq = 0; qq < QW; ++qq) {
          const int row = iw + qq;
          if (row < L) {
            pm[static_cast<int64_t>(row) * g.ldp + jj] = stg[qq * PS + lane];
            gm[static_cast<int64_t>(row) * g.ldp + jj] = stg[(QW + qq) * PS + lane];
          }
        }
      }
    }

    unsigned char *nbuf = smem + ((kt + 1) & 1) * (2 * kLdsT);
    store_kv(nxt, reinterpret_cast<__bf16 *>(nbuf), reinterpret_cast<__bf16 *>(nbuf + kLdsT), tid);
    load_kv(nxt, krs, vrs, kv_row_bytes, j0 + 2 * BK, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// C[z][m][n] (+)= sum_k A_z(m, k) B_z(k, n), n < 64, over the visible part of
// p or g only. Addressing and visibility by kind (jv = first valid key of
// the batch row, c = key index of the element):
//   0  A(m = key j', k = query i)  at a + k*lda + m        visible jv <= m <= M + k
//   1  A(m = query i, k = key j')  at a + m*lda + k        visible jv <= k <= M + m
//   2  A(m = query i, k = row t)   at a + m*lda + c, c = k + m - (L-1)
//   3  A(m = row t, k = query i)   at a + k*lda + c, c = m + k - (L-1), batch row = outer k
// (kinds 2 and 3 are the diagonal view: key c of query i has distance row t).
constexpr int GT = 64;    // output rows per workgroup
constexpr int GK = 64;    // k per slab
constexpr int GS = GK + 8;

struct BgParams {
  int rows, K, K_out, kind;
  const __bf16 *a;
  int64_t lda, a_s1, a_s2, a_so;
  const __bf16 *b;
  int64_t ldb, b_s1, b_s2, b_so;
  float *c;
  int64_t ldc, c_s1, c_s2;
  int accumulate;
  float *colsum;  // optional [z][m tile][64]
  int Z2;
  const int32_t *valid;
  int M, L;
};

// 16 consecutive bf16 of a buffer starting at any element offset off0 (zero
// outside the buffer): three aligned 16-byte loads and a byte-align shift.
__device__ inline void load16_unaligned(rsrc_t rs, int off0, bf16x8 &x0, bf16x8 &x1) {
  const int o = off0 & 7, base8 = off0 - o;
  const u32x4 w0 = bload(rs, 2 * base8), w1 = bload(rs, 2 * base8 + 16), w2 = bload(rs, 2 * base8 + 32);
  const uint32_t win[12] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3],
                            w2[0], w2[1], w2[2], w2[3]};
  const int wsh = o >> 1, sub = (o & 1) * 2;
  u32x4 pk0, pk1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = wsh == 0 ? win[j] : wsh == 1 ? win[j + 1] : wsh == 2 ? win[j + 2] : win[j + 3];
    const uint32_t hi = wsh == 0 ? win[j + 1] : wsh == 1 ? win[j + 2] : wsh == 2 ? win[j + 3] : win[j + 4];
    const uint32_t w = __builtin_amdgcn_alignbyte(hi, lo, sub);
    if (j < 4) pk0[j] = w; else pk1[j - 4] = w;
  }
  x0 = __builtin_bit_cast(bf16x8, pk0);
  x1 = __builtin_bit_cast(bf16x8, pk1);
}

__global__ __launch_bounds__(256) void bgemm_kernel(BgParams q) {
  __shared__ __attribute__((aligned(16))) __bf16 sa[GT * GS];
  __shared__ __attribute__((aligned(16))) __bf16 sb[DH * GS];
  __shared__ float scol[2][DH];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // Workgroups are dealt to the 8 XCDs in turn. When the batch count allows,
  // all row tiles of one z go to the same XCD so that its B operand (the
  // keys, dout, q+u or q+v of that batch row and head) is fetched into one L2
  // instead of eight.
  const int n_mt = (q.rows + GT - 1) / GT;
  const int n_z = static_cast<int>(gridDim.x) / n_mt;
  const int l = static_cast<int>(blockIdx.x);
  int z, mt;
  if ((n_z & 7) == 0) {
    const int w = l >> 3;
    z = (l & 7) + 8 * (w / n_mt);
    mt = w - (w / n_mt) * n_mt;
  } else {
    z = l / n_mt;
    mt = l - z * n_mt;
  }
  const int m0 = mt * GT;
  const int z1 = z / q.Z2, z2 = z - z1 * q.Z2;
  const int M = q.M, L = q.L, ML = M + L;
  const bool trans = q.kind == 0 || q.kind == 3;
  const bool skew = q.kind >= 2;

  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.0f;

  // Each thread moves 16 consecutive elements of A and of B per slab. Where
  // the tile is transposed on its way to LDS (A stored k-major, and every B)
  // the 64 lanes of a wave take 64 consecutive k, so each 2-byte LDS store of
  // the wave touches every bank once or twice.
  const int a_mm = trans ? (tid >> 6) * 16 : tid >> 2;  // m offset in the tile
  const int a_kk = trans ? tid & 63 : (tid & 3) * 16;   // k offset in the slab
  const int b_kk = tid & 63, b_nc = (tid >> 6) * 16;
  // two register sets: the slab being stored to LDS and the next one, so two
  // slabs' loads are in flight while a slab is multiplied
  bf16x8 ra[2][2], rb[2][2];

  for (int ko = 0; ko < q.K_out; ++ko) {
    const int bb = q.K_out > 1 ? ko : z1;      // batch row of the A elements
    int valid = q.valid ? q.valid[bb] : M;
    valid = valid < 0 ? 0 : (valid > M ? M : valid);
    const int jv = M - valid;
    const __bf16 *abase = q.a + (q.K_out > 1 ? ko * q.a_so : z1 * q.a_s1) + z2 * q.a_s2;
    const __bf16 *bbase = q.b + z1 * q.b_s1 + z2 * q.b_s2 + ko * q.b_so;
    const rsrc_t ars = make_rsrc(abase, static_cast<uint32_t>(L * q.lda * 2));
    const int m_last = (m0 + GT < q.rows ? m0 + GT : q.rows) - 1;
    int k_lo = 0, k_hi = q.K;
    if (q.kind == 0) {
      k_lo = m0 - M;
      if (m_last < jv) k_hi = 0;
    } else if (q.kind == 1) {
      k_lo = jv;
      k_hi = M + m_last + 1 < q.K ? M + m_last + 1 : q.K;
    } else {
      k_lo = jv + L - 1 - m_last;
    }
    k_lo = k_lo < 0 ? 0 : (k_lo & ~(GK - 1));
    const int n_slabs = k_hi > k_lo ? (k_hi - k_lo + GK - 1) / GK : 0;

    auto load = [&](int set, int k0) {
      const int m = m0 + a_mm, k = k0 + a_kk;
      // row (query) of the stored matrix and first key / distance of the run
      const int qi = trans ? k : m, t0 = trans ? m : k;
      const int sh = skew ? qi - (L - 1) : 0;         // key = index + sh
      bf16x8 x[2];
      if (!skew) {
        x[0] = x[1] = zero8();
        if (qi < L) {
          const __bf16 *src = abase + static_cast<int64_t>(qi) * q.lda + t0;
          if (t0 < ML) x[0] = load8(src);
          if (t0 + 8 < ML) x[1] = load8(src + 8);
        }
      } else {
        load16_unaligned(ars, qi * static_cast<int>(q.lda) + t0 + sh, x[0], x[1]);
      }
      // visible keys of this query: [jv, M + qi]; indices stay below M + L
      const int k_first = t0 + sh, k_last = t0 + 15 + sh;
      if (qi < L && k_first >= jv && k_last <= M + qi && t0 + 15 < ML) {
        ra[set][0] = x[0];
        ra[set][1] = x[1];
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int idx = t0 + 8 * c + e, key = idx + sh;
            const bool ok = qi < L && idx < ML && key >= jv && key <= M + qi;
            ra[set][c][e] = ok ? x[c][e] : static_cast<__bf16>(0.0f);
          }
      }
      const int kb = k0 + b_kk;
      const __bf16 *bsrc = bbase + static_cast<int64_t>(kb) * q.ldb + b_nc;
      rb[set][0] = kb < q.K ? load8(bsrc) : zero8();
      rb[set][1] = kb < q.K ? load8(bsrc + 8) : zero8();
    };
    auto store = [&](int set) {
      if (trans) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) sa[(a_mm + 8 * c + e) * GS + a_kk] = ra[set][c][e];
      } else {
        *reinterpret_cast<bf16x8 *>(sa + a_mm * GS + a_kk) = ra[set][0];
        *reinterpret_cast<bf16x8 *>(sa + a_mm * GS + a_kk + 8) = ra[set][1];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[(b_nc + 8 * c + e) * GS + b_kk] = rb[set][c][e];
    };
    auto step = [&](int set, int s) {
      __syncthreads();
      store(set);
      __syncthreads();
      if (s + 2 < n_slabs) load(set, k_lo + (s + 2) * GK);
#pragma unroll
      for (int kk = 0; kk < GK / 16; ++kk) {
        const bf16x8 av = load8(sa + (wm * 32 + r) * GS + 16 * kk + 8 * hh);
        const bf16x8 bv = load8(sb + (wn * 32 + r) * GS + 16 * kk + 8 * hh);
        acc = mfma32(av, bv, acc);
      }
    };

    if (n_slabs > 0) load(0, k_lo);
    if (n_slabs > 1) load(1, k_lo + GK);
    for (int s = 0; s < n_slabs; s += 2) {
      step(0, s);
      if (s + 1 < n_slabs) step(1, s + 1);
    }
  }

  float *cp = q.c + z1 * q.c_s1 + z2 * q.c_s2;
  const int n = wn * 32 + r;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int m = m0 + wm * 32 + 8 * (x >> 2) + 4 * hh + (x & 3);
    if (m < q.rows) {
      float *dst = cp + static_cast<int64_t>(m) * q.ldc + n;
      *dst = q.accumulate ? *dst + acc[x] : acc[x];
    }
  }
  if (q.colsum) {
    float s = 0.0f;
#pragma unroll
    for (int x = 0; x < 16; ++x) s += acc[x];  // rows past the end hold zero
    s += __shfl_xor(s, 32);
    if (hh == 0) scol[wm][n] = s;
    __syncthreads();
    if (tid < DH) q.colsum[(static_cast<int64_t>(z) * n_mt + mt) * DH + tid] = scol[0][tid] + scol[1][tid];
  }
}

// dR = sum over batch rows of the per-row products (one thread per element,
// the first 2H workgroups excepted); du[h][n] (dv_bias) = sum over (b, row
// tile) of the column sums of dq's content (position) part, one workgroup
// per (part, head): 4 groups of 64 lanes split the items, then combine.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *part_r, float *dr, int64_t n_r,
                                                         const float *part_u, const float *part_v,
                                                         float *du, float *dvb, int B, int H, int n_mt) {
  __shared__ float red[4][DH];
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) < 2 * H) {
    const int which = static_cast<int>(blockIdx.x) / H, h = static_cast<int>(blockIdx.x) - which * H;
    const float *src = which ? part_v : part_u;
    const int n = tid & 63, grp = tid >> 6, items = B * n_mt;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int it0 = grp; it0 < items; it0 += 16) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int it = it0 + 4 * x;
        if (it < items) {
          const int b = it / n_mt, t = it - b * n_mt;
          acc[x] += src[((static_cast<int64_t>(b) * H + h) * n_mt + t) * DH + n];
        }
      }
    }
    red[grp][n] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (tid < DH) (which ? dvb : du)[h * DH + tid] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    return;
  }
  const int64_t e = (static_cast<int64_t>(blockIdx.x) - 2 * H) * 256 + tid;
  if (e >= n_r) return;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int b0 = 0; b0 < B; b0 += 8) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (b0 + x < B) acc[x] += part_r[(b0 + x) * n_r + e];
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 8; ++x) s += acc[x];
  dr[e] = s;
}

}  // namespace

size_t rel_attn_bwd_ldp(int M, int L) { return (static_cast<size_t>(M) + L + 7) & ~size_t(7); }

txl_status launch_rel_attn_bwd(const AttnParams &p, const BwdParams &g, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_pg_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kLdsTotal)) != hipSuccess)
      return fail(TXL_ERR_HIP, "rel_attn_bwd: cannot raise the LDS limit to %zu bytes", kLdsTotal);
    attr_set = true;
  }
  if (p.kv_sl < DH || p.r_sl < DH || p.q_sl < DH || p.o_sl < DH || g.do_sl < DH)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: bf16 row strides must be >= d_h");
  const int64_t ML = static_cast<int64_t>(p.M) + p.L;
  if ((ML + BK) * p.kv_sl * 2 >= (int64_t(1) << 31) || (ML + BK + QW) * p.r_sl * 2 >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: key / R rows span more than 2 GiB per head");
  if ((static_cast<int64_t>(p.L) * g.ldp + 16) * 2 >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: p / g rows span more than 2 GiB per head");
  const int B = p.B, H = p.H, L = p.L;
  const int64_t BHL = static_cast<int64_t>(B) * H * L;
  const int n_qt = (L + BQ - 1) / BQ;
  const int64_t blocks = static_cast<int64_t>(n_qt) * B * H;
  if (blocks > 0x7fffffffLL || BHL * 8 / 256 + 1 > 0x7fffffffLL)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: grid too large");
  (void)hipGetLastError();
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((BHL * 8 + 255) / 256)), dim3(256), 0, s,
                     p, g);
  txl_status st = check_launch("bwd_prep_kernel");
  if (st != TXL_OK) return st;
  hipLaunchKernelGGL(bwd_pg_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), kLdsTotal, s, p, g, n_qt);
  if ((st = check_launch("bwd_pg_kernel")) != TXL_OK) return st;

  const int ml = static_cast<int>(ML);
  auto run = [&](BgParams q, int z_count) -> txl_status {
    q.valid = p.valid;
    q.M = p.M;
    q.L = L;
    const int64_t wgs = static_cast<int64_t>((q.rows + GT - 1) / GT) * z_count;
    hipLaunchKernelGGL(bgemm_kernel, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, s, q);
    return check_launch("bgemm_kernel");
  };
  const int64_t pz = static_cast<int64_t>(L) * g.ldp;      // p / g per (b, h)
  const int n_mt_q = (L + GT - 1) / GT;

  BgParams q = {};
  // dv = p^T dout
  q.rows = ml; q.K = L; q.K_out = 1; q.kind = 0;
  q.a = g.pm; q.lda = g.ldp; q.a_s1 = H * pz; q.a_s2 = pz;
  q.b = g.dout; q.ldb = g.do_sl; q.b_s1 = g.do_sb; q.b_s2 = g.do_sh;
  q.c = g.dv; q.ldc = DH; q.c_s1 = static_cast<int64_t>(H) * ml * DH; q.c_s2 = static_cast<int64_t>(ml) * DH;
  q.Z2 = H;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  // dk = g^T (q + u)
  q.a = g.gm;
  q.b = g.qu; q.ldb = DH; q.b_s1 = static_cast<int64_t>(H) * L * DH; q.b_s2 = static_cast<int64_t>(L) * DH;
  q.c = g.dk;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  // dq = g k (content part) ...
  q = BgParams{};
  q.rows = L; q.K = ml; q.K_out = 1; q.kind = 1;
  q.a = g.gm; q.lda = g.ldp; q.a_s1 = H * pz; q.a_s2 = pz;
  q.b = static_cast<const __bf16 *>(p.k); q.ldb = p.kv_sl; q.b_s1 = p.kv_sb; q.b_s2 = p.kv_sh;
  q.c = g.dq; q.ldc = DH; q.c_s1 = static_cast<int64_t>(H) * L * DH; q.c_s2 = static_cast<int64_t>(L) * DH;
  q.colsum = g.part_u; q.Z2 = H;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  // ... + g R over the diagonal view (position part)
  q.kind = 2;
  q.b = static_cast<const __bf16 *>(p.r); q.ldb = p.r_sl; q.b_s1 = 0; q.b_s2 = p.r_sh;
  q.accumulate = 1; q.colsum = g.part_v;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  // dR per batch row = sum over queries of g (q + v), diagonal view; summed
  // over batch rows by the reduction below
  q = BgParams{};
  q.rows = ml; q.K = L; q.K_out = 1; q.kind = 3;
  q.a = g.gm; q.lda = g.ldp; q.a_s1 = H * pz; q.a_s2 = pz;
  q.b = g.qv; q.ldb = DH; q.b_s1 = static_cast<int64_t>(H) * L * DH; q.b_s2 = static_cast<int64_t>(L) * DH;
  q.c = g.part_r; q.ldc = DH; q.c_s1 = static_cast<int64_t>(H) * ml * DH; q.c_s2 = static_cast<int64_t>(ml) * DH;
  q.Z2 = H;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  const int64_t n_r = static_cast<int64_t>(H) * ml * DH;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>(2 * H + (n_r + 255) / 256)), dim3(256), 0, s,
                     g.part_r, g.dr, n_r, g.part_u, g.part_v, g.du, g.dvb, B, H, n_mt_q);
  return check_launch("bwd_reduce_kernel");
}

}  // namespace txl
