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
// Design:
//  * bwd_prep: D_i, and (q+v) rounded to bf16 for the dR product.
//  * bwd_kv: key-major. A workgroup holds 128 keys of one (batch, head); each
//    wave keeps its 32 K and V rows and its dK, dV accumulators in registers
//    while query tiles of 32 stream through LDS. Per tile it recomputes the
//    scores as the forward does (content MFMA, the position band and its
//    diagonal read through LDS), forms p = 2^(s - lse) from the forward's
//    log-sum-exp, dp = dout V^T and g = scale p (dp - D), and accumulates
//    dV += p^T dout and dK += g^T (q+u) on the chip. g leaves twice, as bf16
//    rows by key, g[i][j'], and by distance, g[i][t] with t = j' + L - 1 - i
//    (consecutive lanes write consecutive keys of a row in both).
//  * bgemm: one small MFMA kernel for the remaining contractions, reading the
//    visible part of each row only (hidden entries are masked on load, so
//    nothing outside the visited pairs needs clearing): dq = g K over keys,
//    dq += g R over distances, dR = sum over queries of g (q + v) per batch
//    row.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int DH = 64;
constexpr int NW = 4;          // waves per workgroup

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
// 2-byte store; offsets past the buffer's end are dropped by the range check
__device__ inline void bstore16(__bf16 v, rsrc_t rs, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rs, voff, soff, 0);
}
constexpr int kDropOffset = 0x40000000;   // past any p / g slice (slices stay below 1 GiB)

// ---------------------------------------------------------------------------
// D_i = dout_i . out_i (fp32; out unrounded when the forward kept it) and
// qv = bf16(q + v) (the dR product's operand); one thread per query row and
// 8 dimensions.
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
    const bf16x8 vv = load8(static_cast<const __bf16 *>(p.vb) + h * DH + 8 * c);
    float of[8];
    if (g.out32) {  // the unrounded output, when the forward kept it
      const f32x4 lo = *reinterpret_cast<const f32x4 *>(g.out32 + row * DH + 8 * c);
      const f32x4 hi = *reinterpret_cast<const f32x4 *>(g.out32 + row * DH + 8 * c + 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        of[x] = lo[x];
        of[x + 4] = hi[x];
      }
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) of[x] = static_cast<float>(ov[x]);
    }
    bf16x8 bq;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      bq[x] = static_cast<__bf16>(static_cast<float>(qv[x]) + static_cast<float>(vv[x]));
      acc += static_cast<float>(dv[x]) * of[x];
    }
    *reinterpret_cast<bf16x8 *>(g.qv + row * DH + 8 * c) = bq;
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < BHL && c == 0) g.dd[row] = acc;
}

// ---------------------------------------------------------------------------
// Key-major pass: one workgroup = 4 waves x 32 keys of one (batch, head); each
// wave keeps its K and V rows (MFMA B operands) and its dK^T, dV^T
// accumulators in registers while query tiles of 32 stream through LDS.
// Per query tile, in the [query][key] accumulator layout (lane = key):
//   S = Q' K^T (+ the position band Q'' R^T read along its diagonal through
//   LDS), p = 2^(S - lse2), dp = dout V^T, g = scale p (dp - D),
//   dV^T += dout^T p, dK^T += (q+u)^T g  (k-order of the query index matching
//   the accumulator rows, as the forward's PV product),
// and g goes out twice: by key, g[i][j'], and by distance, g[i][t] with
// t = j' + L - 1 - i (both rows written by consecutive lanes).
constexpr int KW = 32;            // keys per wave
constexpr int KB2 = KW * NW;      // keys per workgroup
constexpr int QT = 32;            // queries per tile
constexpr int TS = DH + 8;        // Q' / Q'' / dout tile row stride (bf16)
constexpr int TT = QT + 4;        // transposed tile row stride (bf16): 8-byte rows, 4-way at most
constexpr int BS = 2 * QT + 4;    // band row stride (floats): [query][u], u < 64
constexpr size_t kKvLdsTile = size_t(QT) * TS * 2;          // one [32][72] bf16 tile
constexpr size_t kKvLdsTr = size_t(DH) * TT * 2;            // one [64][40] bf16 tile
constexpr size_t kKvLdsBand = size_t(NW) * QT * BS * 4;
constexpr size_t kKvLdsTotal = 3 * kKvLdsTile + 2 * kKvLdsTr + 2 * QT * 4 + kKvLdsBand + 2 * DH * 2;

// Dims 4 c4 .. 4 c4 + 3 of key j's dK and dV (batch row b, head h): fp32
// per head where dkp / dvp are set, and the bf16 rows of g.rows.
__device__ inline void store_kv_grad(const BwdParams &g, float *dkp, float *dvp, int b, int h, int ML,
                                     int M, int L, int j, int c4, f32x4 dk, f32x4 dv) {
  if (dkp) *reinterpret_cast<f32x4 *>(dkp + static_cast<int64_t>(j) * DH + 4 * c4) = dk;
  if (dvp) *reinterpret_cast<f32x4 *>(dvp + static_cast<int64_t>(j) * DH + 4 * c4) = dv;
  bf16x4 kb4, vb4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kb4[e] = static_cast<__bf16>(dk[e]);
    vb4[e] = static_cast<__bf16>(dv[e]);
  }
  const int col = h * DH + 4 * c4;
  const int64_t row = static_cast<int64_t>(b) * ML + j;
  if (g.rows.dk) *reinterpret_cast<bf16x4 *>(g.rows.dk + row * g.rows.kv_ld + col) = kb4;
  if (g.rows.dv) *reinterpret_cast<bf16x4 *>(g.rows.dv + row * g.rows.kv_ld + col) = vb4;
  if (j >= M) {
    const int64_t srow = static_cast<int64_t>(b) * L + (j - M);
    if (g.rows.dk_seg) *reinterpret_cast<bf16x4 *>(g.rows.dk_seg + srow * g.rows.seg_ld + col) = kb4;
    if (g.rows.dv_seg) *reinterpret_cast<bf16x4 *>(g.rows.dv_seg + srow * g.rows.seg_ld + col) = vb4;
  }
}

__global__ __launch_bounds__(256, 2) void bwd_kv_kernel(AttnParams p, BwdParams g, int n_kb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16 *sQa = reinterpret_cast<__bf16 *>(smem);
  __bf16 *sQb = sQa + QT * TS;
  __bf16 *sDo = sQb + QT * TS;
  __bf16 *sQuT = sDo + QT * TS;            // [64 dims][32 queries]
  __bf16 *sDoT = sQuT + DH * TT;
  float *sLse = reinterpret_cast<float *>(sDoT + DH * TT);
  float *sD = sLse + QT;
  float *sband = sD + QT;
  __bf16 *sUV = reinterpret_cast<__bf16 *>(sband + NW * QT * BS);  // u [64] then v [64]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int BH = p.B * p.H;
  const int kb = static_cast<int>(blockIdx.x) / BH;       // key blocks in order: most queries first
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int L = p.L, M = p.M, ML = M + L;
  const int jb = kb * KB2, jw = jb + wave * KW, j = jw + r;   // this lane's key

  int valid = p.valid ? p.valid[b] : M;
  valid = valid < 0 ? 0 : (valid > M ? M : valid);
  const int jv = M - valid;

  const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16 *kp = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *vp = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *rp = static_cast<const __bf16 *>(p.r) + h * p.r_sh;
  const __bf16 *up = static_cast<const __bf16 *>(p.u) + h * DH;
  const __bf16 *vbp = static_cast<const __bf16 *>(p.vb) + h * DH;
  const __bf16 *dop = g.dout + b * g.do_sb + h * g.do_sh;
  const int64_t row_bh = static_cast<int64_t>(bh) * L;
  float *dkp = g.dk ? g.dk + static_cast<int64_t>(bh) * ML * DH : nullptr;
  float *dvp = g.dv ? g.dv + static_cast<int64_t>(bh) * ML * DH : nullptr;
  float *band = sband + wave * (QT * BS);

  // keys below the first valid one, or past the last, take no gradient; a
  // block of only such keys writes zeros and stops
  const int q_first = jb + KB2 - 1 < M ? 0 : ((jb - M > 0 ? jb - M : 0) & ~(QT - 1));
  if (jb + KB2 - 1 < jv || q_first >= L) {
    for (int e = tid; e < KB2 * DH / 4; e += 256) {
      const int kk = e / (DH / 4), c4 = e - kk * (DH / 4);
      if (jb + kk < ML) {
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        store_kv_grad(g, dkp, dvp, b, h, ML, M, L, jb + kk, c4, z, z);
      }
    }
    return;
  }

  // K and V rows of this lane's key as B operands (zero past the end)
  bf16x8 kreg[4], vreg[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int d0 = 16 * s + 8 * hh;
    kreg[s] = j < ML ? load8(kp + static_cast<int64_t>(j) * p.kv_sl + d0) : zero8();
    vreg[s] = j < ML ? load8(vp + static_cast<int64_t>(j) * p.kv_sl + d0) : zero8();
  }
  const int r_row_bytes = static_cast<int>(p.r_sl) * 2;
  const rsrc_t rrs = make_rsrc(rp, static_cast<uint32_t>((ML - 1) * r_row_bytes + 2 * DH));

  // query-tile staging: thread -> (query row, 8-dim chunk)
  const int st_row = tid >> 3, st_c = (tid & 7) * 8;
  const float c2 = p.scale * 1.4426950408889634f;
  // The next query tile's loads are issued unconditionally (rows past L
  // read row L-1) and nothing is computed from them before stage(): with
  // the loads behind branches, or scaled right after loading, the compiler
  // waited for them (and so for every load before them) at once.
  bf16x8 nq, ndo;
  float nlse = 0.0f, nd = 0.0f;
  bool nq_ok = false, nl_ok = false;
  auto fetch = [&](int i0) {
    const int i = i0 + st_row;
    nq_ok = i < L;
    const int64_t ic = nq_ok ? i : L - 1;
    nq = load8(qp + ic * p.q_sl + st_c);
    ndo = load8(dop + ic * g.do_sl + st_c);
    const int ii = i0 + (tid & (QT - 1));
    nl_ok = ii < L;
    const int64_t iic = nl_ok ? ii : L - 1;
    nlse = g.lse[row_bh + iic];
    nd = g.dd[row_bh + iic];
  };
  // u and v of the head, read by every stage, sit in LDS (written before
  // the first stage's barrier)
  if (tid < 16) *reinterpret_cast<bf16x8 *>(sUV + 8 * tid) = load8((tid < 8 ? up : vbp) + 8 * (tid & 7));
  auto stage = [&]() {
    const bf16x8 u8 = *reinterpret_cast<const bf16x8 *>(sUV + st_c);
    const bf16x8 v8 = *reinterpret_cast<const bf16x8 *>(sUV + DH + st_c);
    if (!nq_ok) {
      nq = zero8();
      ndo = zero8();
    }
    bf16x8 a, bq, qu;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = static_cast<float>(nq[e]);
      const float xu = x + static_cast<float>(u8[e]);
      a[e] = static_cast<__bf16>(xu * c2);
      bq[e] = static_cast<__bf16>((x + static_cast<float>(v8[e])) * c2);
      qu[e] = static_cast<__bf16>(xu);
    }
    *reinterpret_cast<bf16x8 *>(sQa + st_row * TS + st_c) = a;
    *reinterpret_cast<bf16x8 *>(sQb + st_row * TS + st_c) = bq;
    *reinterpret_cast<bf16x8 *>(sDo + st_row * TS + st_c) = ndo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sQuT[(st_c + e) * TT + st_row] = qu[e];
      sDoT[(st_c + e) * TT + st_row] = ndo[e];
    }
    if (tid < QT) {
      sLse[tid] = nl_ok ? nlse * 1.4426950408889634f : 0.0f;
      sD[tid] = nl_ok ? nd * p.scale : 0.0f;   // scale * D
    }
  };

  // g by key: element (i, j) at byte (i*ldp + j)*2 of the (b, h) slice; by
  // distance: (i, j + L-1-i) at byte (i*(ldp-1) + j + L-1)*2. The lane part of
  // the offset is in voff, the register's row part (a multiple of the row
  // stride) in soff; hidden keys and lanes past the end use kDropOffset.
  const uint32_t slice_bytes = static_cast<uint32_t>(static_cast<int64_t>(L) * g.ldp * 2);
  const rsrc_t grs = make_rsrc(g.gm + row_bh * g.ldp, slice_bytes);
  const rsrc_t srs = make_rsrc(g.pm + row_bh * g.ldp, slice_bytes);
  const int ldp = static_cast<int>(g.ldp);
  const bool j_ok = j >= jv && j < ML;
  const bool tile_keys_visible = jw >= jv && jw + KW - 1 < ML;

  f32x16 dv_acc[2], dk_acc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) dv_acc[db][x] = dk_acc[db][x] = 0.0f;

  // R rows of the band: for query tile i0 the band columns are t0 + 0..63,
  // t0 = jw + L - 1 - i0 - 31; column block c holds R rows t0 + 32c + r
  auto load_rblk = [&](bf16x8 (&dst)[4], int t_first) {
    const int off = (t_first + r) * r_row_bytes + 16 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = __builtin_bit_cast(bf16x8, bload(rrs, off + 32 * s));
  };
  bf16x8 rb0[4], rb1[4];
  load_rblk(rb0, jw + L - 1 - q_first - 31);
  load_rblk(rb1, jw + L - 1 - q_first - 31 + 32);

  fetch(q_first);
  __syncthreads();
  stage();
  __syncthreads();
  const float scale = p.scale;
  for (int i0 = q_first; i0 < L; i0 += QT) {
    fetch(i0 + QT);  // past the last tile: loaded, never staged

    // ---- the band Q'' R^T, one 32-column block at a time, to LDS as
    // band[q][u] (u = t - t0); the next tile's band starts 32 rows lower, so
    // its block 1 is this block 0 ----
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x16 bacc;
#pragma unroll
      for (int x = 0; x < 16; ++x) bacc[x] = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        bacc = mfma32(load8(sQb + r * TS + 16 * s + 8 * hh), c == 0 ? rb0[s] : rb1[s], bacc);
#pragma unroll
      for (int x = 0; x < 16; ++x) band[(8 * (x >> 2) + 4 * hh + (x & 3)) * BS + 32 * c + r] = bacc[x];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) rb1[s] = rb0[s];
    if (i0 + QT < L) load_rblk(rb0, jw + L - 1 - (i0 + QT) - 31);
    // ---- S[q][key] = Q' K^T, plus S_pos[q][key] = band[q][key - q + 31] ----
    f32x16 sacc;
#pragma unroll
    for (int x = 0; x < 16; ++x) sacc[x] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) sacc = mfma32(load8(sQa + r * TS + 16 * s + 8 * hh), kreg[s], sacc);
    wave_lds_sync();
    float sv[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int qq = 8 * (x >> 2) + 4 * hh + (x & 3);
      sv[x] = sacc[x] + band[qq * BS + r + 31 - qq];
    }
    wave_lds_sync();

    // ---- dp[q][key] = dout V^T ----
    f32x16 dpa;
#pragma unroll
    for (int x = 0; x < 16; ++x) dpa[x] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) dpa = mfma32(load8(sDo + r * TS + 16 * s + 8 * hh), vreg[s], dpa);

    // ---- p and g; masked pairs (hidden key, future key, query past the end)
    // get 0; a tile whose pairs are all visible skips the test ----
    bf16x8 pb[2], gb[2];
    const bool all_vis = tile_keys_visible && i0 + QT <= L && jw + KW - 1 - M <= i0;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sLse + 8 * a4 + 4 * hh);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sD + 8 * a4 + 4 * hh);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int x = 4 * a4 + c;
        const int i = i0 + 8 * a4 + 4 * hh + c;
        const bool vis = all_vis || (i < L && j_ok && j - M <= i);
        // a select on the argument (2^-inf = 0), not a branch around the exp
        const float pv = __builtin_amdgcn_exp2f(vis ? sv[x] - l4[c] : -INFINITY);
        const float gg = pv * (dpa[x] * scale - d4[c]);
        pb[x >> 3][x & 7] = static_cast<__bf16>(pv);
        gb[x >> 3][x & 7] = static_cast<__bf16>(gg);
      }
    }

    // ---- dV^T += dout^T p, dK^T += (q+u)^T g: k-step s2 covers queries
    // 16 s2 + {4hh..4hh+3, 8+4hh..8+4hh+3} ----
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int o = (db * 32 + r) * TT + 16 * s2 + 4 * hh;
        const bf16x4 dlo = *reinterpret_cast<const bf16x4 *>(sDoT + o);
        const bf16x4 dhi = *reinterpret_cast<const bf16x4 *>(sDoT + o + 8);
        const bf16x4 ulo = *reinterpret_cast<const bf16x4 *>(sQuT + o);
        const bf16x4 uhi = *reinterpret_cast<const bf16x4 *>(sQuT + o + 8);
        bf16x8 ad, au;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ad[e] = dlo[e];
          ad[e + 4] = dhi[e];
          au[e] = ulo[e];
          au[e + 4] = uhi[e];
        }
        dv_acc[db] = mfma32(ad, pb[s2], dv_acc[db]);
        dk_acc[db] = mfma32(au, gb[s2], dk_acc[db]);
      }

    // ---- g by key and by distance (rows of consecutive keys); rows past L
    // fall outside the slice and are dropped ----
    {
      const int ih = i0 + 4 * hh;   // this lane half's first row (+ 8 a4 + c)
      const int vg = j < ML ? (ih * ldp + j) * 2 : kDropOffset;
      const int vs = (ih * (ldp - 1) + j + L - 1) * 2;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int rr = 8 * (x >> 2) + (x & 3);   // row offset common to the wave
        const __bf16 gbv = gb[x >> 3][x & 7];
        bstore16(gbv, grs, vg, rr * ldp * 2);
        // (by distance, a row past L can map back into the slice: test it)
        const bool vis = all_vis || (j_ok && j - M <= ih + rr && ih + rr < L);
        bstore16(gbv, srs, vis ? vs : kDropOffset, rr * (ldp - 1) * 2);
      }
    }

    __syncthreads();   // every wave is done with this tile's LDS
    if (i0 + QT < L) stage();
    __syncthreads();
  }

  // ---- dK, dV rows through LDS (this wave's band area, one after the
  // other), four dims of a key a lane, then stored together ----
  float *st = band;   // [32 keys][64 + 4 dims]
  static_assert(size_t(KW) * (DH + 4) * 4 <= size_t(QT) * BS * 4, "dK / dV staging must fit a wave's band");
  constexpr int NIT = KW * DH / 4 / 64;
  f32x4 kv4[2][NIT];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int dh = db * 32 + 8 * (x >> 2) + 4 * hh + (x & 3);
        st[r * (DH + 4) + dh] = pass == 0 ? dk_acc[db][x] : dv_acc[db][x];
      }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e = lane + 64 * it;
      const int kk = e / (DH / 4), c4 = e - kk * (DH / 4);
      kv4[pass][it] = *reinterpret_cast<const f32x4 *>(st + kk * (DH + 4) + 4 * c4);
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = lane + 64 * it;
    const int kk = e / (DH / 4), c4 = e - kk * (DH / 4);
    if (jw + kk < ML) store_kv_grad(g, dkp, dvp, b, h, ML, M, L, jw + kk, c4, kv4[0][it], kv4[1][it]);
  }
  (void)n_kb;
}

// ---------------------------------------------------------------------------
// C[z][m][n] (+)= sum_k A_z(m, k) B_z(k, n), n < 64, over the visible part of
// g only. A is g stored by key or by distance, element (i, c) of query i at
// a + i*lda + c; addressing and visibility by kind (jv = first valid key of
// the batch row):
//   1  A(m = query i, k = key j')  = g_key(i, k)     visible jv <= k <= M + m
//   2  A(m = query i, k = row t)   = g_dist(i, k)    key t + m - (L-1) visible
//   3  A(m = row t, k = query i)   = g_dist(k, m)    key m + k - (L-1) visible
// (kinds 2 and 3 are the diagonal view: distance row t of query i is key
// t + i - (L-1)).
constexpr int GT = 64;    // output rows per workgroup
constexpr int GK = 64;    // k per slab
constexpr int GS = GK + 8;

// One operand set of a product: C += A B over K, A addressed by kind.
struct BgPhase {
  int kind, K;
  const __bf16 *a;
  int64_t lda, a_s1, a_s2;
  const __bf16 *b;
  int64_t ldb, b_s1, b_s2;
  float *colsum;  // optional [z][m tile][64]: column sums of this phase's share of C
};
// C = sum over phases (one or two, sharing the output rows) of A B.
struct BgParams {
  int rows, n_phase;
  BgPhase ph[2];
  float *c;
  __bf16 *c16;      // bf16 output instead of c when set (same strides)
  int64_t ldc, c_s1, c_s2;
  int Z2;
  const int32_t *valid;
  int M, L;
};

// k-major LDS tiles ([k][64], 128-byte rows): the 16-byte chunk c of row k
// sits in slot c ^ (4 * ((k >> 1) & 1)), so that the transposing operand
// read (four rows of 64 bytes for 32 lanes) covers every bank once
__device__ inline int kmaj_off(int row, int col) {
  return row * 64 + 8 * ((col >> 3) ^ (((row >> 1) & 1) << 2)) + (col & 7);
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
// Transposing LDS read: within each 16-lane group, element k of lane j is the
// 16-bit value at (address of lane 4k + j/4) + j % 4.
__device__ inline v4i16 lds_read_tr(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
}

__global__ __launch_bounds__(256) void bgemm_kernel(BgParams q) {
  __shared__ __attribute__((aligned(16))) __bf16 sa[GT * GS];   // [m][k] padded, or k-major
  __shared__ __attribute__((aligned(16))) __bf16 sb[GK * DH];   // k-major
  __shared__ float scol[2][DH];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // Workgroups are dealt to the 8 XCDs in turn. When the batch count allows,
  // all row tiles of one z go to the same XCD so that its B operand (the
  // keys, R or q+v of that batch row and head) is fetched into one L2
  // instead of eight.
  const int n_mt = (q.rows + GT - 1) / GT;
  const int n_z = static_cast<int>(gridDim.x) / n_mt;
  const int l = static_cast<int>(blockIdx.x);
  int z, mt;
  if ((n_z & 7) == 0) {
    const int w = l >> 3;
    z = (l & 7) + 8 * (w / n_mt);
    mt = w - (w / n_mt) * n_mt;
    // Rows see triangular key ranges (the last row tile about twice the keys
    // of the first), and an XCD deals its workgroups to its 32 CUs in turn,
    // so CU c would receive row tile c mod n_mt in every round. Every other
    // round of 32 takes the row tiles in reverse, so a CU holds tiles mt and
    // n_mt - 1 - mt alike. (Only where n_mt divides 32, so that one batch
    // row's tiles stay within one round and the mapping stays one-to-one.)
    if ((32 % n_mt) == 0 && ((w >> 5) & 1)) mt = n_mt - 1 - mt;
  } else {
    z = l / n_mt;
    mt = l - z * n_mt;
  }
  const int m0 = mt * GT;
  const int z1 = z / q.Z2, z2 = z - z1 * q.Z2;
  const int M = q.M, L = q.L;
  int valid = q.valid ? q.valid[z1] : M;
  valid = valid < 0 ? 0 : (valid > M ? M : valid);
  const int jv = M - valid;
  const int m_last = (m0 + GT < q.rows ? m0 + GT : q.rows) - 1;
  const int n = wn * 32 + r;

  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.0f;
  float col_before = 0.0f;   // this lane's column sum before the phase

  // Operand reads of the k-major tiles: lane 16g + 4kq + jq supplies the
  // address of row 8(g >> 1) + kq (+ 16 per k-step, + 4 for the second four
  // k) at column c0 + 16(g & 1) + 4jq, so that lane j of its group receives
  // the column's four k in a row: a lane gets k = 8hh .. 8hh + 7 of column
  // c0 + r, the operand layout of the MFMA (c0 = 32 wm for A, 32 wn for B).
  int tr_a, tr_b;
  {
    const int g = lane >> 4, kq = (lane >> 2) & 3, jq = lane & 3;
    tr_a = kmaj_off(8 * (g >> 1) + kq, 32 * wm + 16 * (g & 1) + 4 * jq);
    tr_b = kmaj_off(8 * (g >> 1) + kq, 32 * wn + 16 * (g & 1) + 4 * jq);
  }

  // two register sets: the slab being stored to LDS and the next one, so two
  // slabs' loads are in flight while a slab is multiplied. The loads are
  // issued unconditionally (A range-checked, B at a clamped row) and their
  // registers are not read before the slab is stored two steps later, where
  // the hidden entries are zeroed: so the compiler's count of loads in flight
  // stays exact and a step waits only for the slab it stores.
  u32x4 xa[2][2];
  bf16x8 rb[2][2];

  for (int ph = 0; ph < q.n_phase; ++ph) {
    const BgPhase &P = q.ph[ph];
    const bool trans = P.kind == 3;             // A read k-major (by query)
    const bool skew = P.kind >= 2;              // indexed by distance: key = t + i - (L-1)
    // Each thread moves 16 consecutive elements of one stored row of A and of
    // B per slab (four threads per 128-byte row). A stored by query (kind 3)
    // and every B are kept k-major in LDS and read through the transposing
    // operand read; the others keep A m-major, read 16 bytes at a time.
    const int a_mm = trans ? (tid & 3) * 16 : tid >> 2;   // m offset in the tile
    const int a_kk = trans ? tid >> 2 : (tid & 3) * 16;   // k offset in the slab
    const int b_kk = tid >> 2, b_nc = (tid & 3) * 16;
    const __bf16 *abase = P.a + z1 * P.a_s1 + z2 * P.a_s2;
    const __bf16 *bbase = P.b + z1 * P.b_s1 + z2 * P.b_s2;
    const rsrc_t ars = make_rsrc(abase, static_cast<uint32_t>(L * P.lda * 2));
    int k_lo = 0, k_hi = P.K;
    if (P.kind == 1) {
      k_lo = jv;
      k_hi = M + m_last + 1 < P.K ? M + m_last + 1 : P.K;
    } else {
      k_lo = jv + L - 1 - m_last;
    }
    k_lo = k_lo < 0 ? 0 : (k_lo & ~(GK - 1));
    const int n_slabs = k_hi > k_lo ? (k_hi - k_lo + GK - 1) / GK : 0;
    const int k_last_slab = k_lo + (n_slabs > 0 ? n_slabs - 1 : 0) * GK;

    // slabs past the last are read again as the last (cache hits, never stored)
    auto load = [&](int set, int k0) {
      k0 = k0 < k_last_slab ? k0 : k_last_slab;
      const int m = m0 + a_mm, k = k0 + a_kk;
      const int qi = trans ? k : m, t0 = trans ? m : k;
      // rows at or past L fall outside the range and read as zeros; entries
      // past M + L - 1 of a row are hidden and zeroed at the store
      const int off = 2 * ((qi < L ? qi : L) * static_cast<int>(P.lda) + t0);
      xa[set][0] = bload(ars, off);
      xa[set][1] = bload(ars, off + 16);
      const int kb = k0 + b_kk;
      const __bf16 *bsrc = bbase + static_cast<int64_t>(kb < P.K ? kb : P.K - 1) * P.ldb + b_nc;
      rb[set][0] = load8(bsrc);
      rb[set][1] = load8(bsrc + 8);
    };
    auto store = [&](int set, int k0) {
      const int m = m0 + a_mm, k = k0 + a_kk;
      const int qi = trans ? k : m, t0 = trans ? m : k;
      const int sh = skew ? qi - (L - 1) : 0;         // key = index + sh
      bf16x8 x[2] = {__builtin_bit_cast(bf16x8, xa[set][0]), __builtin_bit_cast(bf16x8, xa[set][1])};
      // visible keys of this query: [jv, M + qi]; indices stay below M + L
      const int k_first = t0 + sh, k_last = t0 + 15 + sh;
      if (!(qi < L && k_first >= jv && k_last <= M + qi && t0 + 15 < M + L)) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int idx = t0 + 8 * c + e, key = idx + sh;
            const bool ok = qi < L && idx < M + L && key >= jv && key <= M + qi;
            x[c][e] = ok ? x[c][e] : static_cast<__bf16>(0.0f);
          }
      }
      if (trans) {
        *reinterpret_cast<bf16x8 *>(sa + kmaj_off(a_kk, a_mm)) = x[0];
        *reinterpret_cast<bf16x8 *>(sa + kmaj_off(a_kk, a_mm + 8)) = x[1];
      } else {
        *reinterpret_cast<bf16x8 *>(sa + a_mm * GS + a_kk) = x[0];
        *reinterpret_cast<bf16x8 *>(sa + a_mm * GS + a_kk + 8) = x[1];
      }
      const bool b_ok = k0 + b_kk < P.K;
      *reinterpret_cast<bf16x8 *>(sb + kmaj_off(b_kk, b_nc)) = b_ok ? rb[set][0] : zero8();
      *reinterpret_cast<bf16x8 *>(sb + kmaj_off(b_kk, b_nc + 8)) = b_ok ? rb[set][1] : zero8();
    };
    auto step = [&](int set, int s) {
      __syncthreads();
      store(set, k_lo + s * GK);
      __syncthreads();
      load(set, k_lo + (s + 2) * GK);
#pragma unroll
      for (int kk = 0; kk < GK / 16; ++kk) {
        bf16x8 av;
        if (trans) {
          const v4i16 lo = lds_read_tr(sa + tr_a + 1024 * kk), hi = lds_read_tr(sa + tr_a + 1024 * kk + 256);
          av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          av = load8(sa + (wm * 32 + r) * GS + 16 * kk + 8 * hh);
        }
        const v4i16 lo = lds_read_tr(sb + tr_b + 1024 * kk), hi = lds_read_tr(sb + tr_b + 1024 * kk + 256);
        // one cast of the whole vector (a per-element cast of the halves is
        // folded wrongly by the compiler)
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc = mfma32(av, bv, acc);
      }
    };

    // both steps of every iteration run (an odd slab count ends with one
    // more step after the loop), and the loop is entered only after the two
    // first loads, so every step is entered with the same loads in flight
    if (n_slabs > 0) {
      load(0, k_lo);
      load(1, k_lo + GK);
      int s2 = 0;
      for (; s2 + 1 < n_slabs; s2 += 2) {
        step(0, s2);
        step(1, s2 + 1);
      }
      if (s2 < n_slabs) step(0, s2);
    }

    if (P.colsum) {   // (uniform) this phase's share of the column sums
      float sum = 0.0f;
#pragma unroll
      for (int x = 0; x < 16; ++x) sum += acc[x];  // rows past the end hold zero
      sum += __shfl_xor(sum, 32);
      const float share = sum - col_before;
      col_before = sum;
      __syncthreads();   // scol of an earlier phase has been read
      if (hh == 0) scol[wm][n] = share;
      __syncthreads();
      if (tid < DH) P.colsum[(static_cast<int64_t>(z) * n_mt + mt) * DH + tid] = scol[0][tid] + scol[1][tid];
    }
  }

  const int64_t co = z1 * q.c_s1 + z2 * q.c_s2;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int m = m0 + wm * 32 + 8 * (x >> 2) + 4 * hh + (x & 3);
    if (m < q.rows) {
      if (q.c16)
        q.c16[co + static_cast<int64_t>(m) * q.ldc + n] = static_cast<__bf16>(acc[x]);
      else
        q.c[co + static_cast<int64_t>(m) * q.ldc + n] = acc[x];
    }
  }
}

// dR = sum over batch rows of the per-row products (one thread per element,
// the first 2H workgroups excepted); du[h][n] (dv_bias) = sum over (b, row
// tile) of the column sums of dq's content (position) part, one workgroup
// per (part, head): 4 groups of 64 lanes split the items, then combine.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *part_r, float *dr, int64_t n_r,
                                                         const float *part_u, const float *part_v,
                                                         float *du, float *dvb, int B, int H, int n_mt,
                                                         __bf16 *dr_rows, int64_t dr_ld, int ml) {
  __shared__ float red[4][DH];
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) < 2 * H) {
    const int which = static_cast<int>(blockIdx.x) / H, h = static_cast<int>(blockIdx.x) - which * H;
    const float *src = which ? part_v : part_u;
    const int n = tid & 63, grp = tid >> 6, items = B * n_mt;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // the four items of a round are loaded before any is added (items past
    // the end load the last item and add nothing): loads behind the item
    // test were waited for one at a time
    for (int it0 = grp; it0 < items; it0 += 16) {
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int it = it0 + 4 * x < items ? it0 + 4 * x : items - 1;
        const int b = it / n_mt, t = it - b * n_mt;
        v[x] = src[((static_cast<int64_t>(b) * H + h) * n_mt + t) * DH + n];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (it0 + 4 * x < items) acc[x] += v[x];
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
    float v[8];  // loaded together, as above
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = part_r[(b0 + x < B ? b0 + x : B - 1) * n_r + e];
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (b0 + x < B) acc[x] += v[x];
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 8; ++x) s += acc[x];
  if (dr) dr[e] = s;
  if (dr_rows) {  // e = (h (M+L) + t) 64 + n  ->  row t, column h 64 + n
    const int64_t ht = e / DH;
    const int n = static_cast<int>(e - ht * DH);
    const int hh2 = static_cast<int>(ht / ml), t = static_cast<int>(ht - static_cast<int64_t>(hh2) * ml);
    dr_rows[static_cast<int64_t>(t) * dr_ld + hh2 * DH + n] = static_cast<__bf16>(s);
  }
}

}  // namespace

size_t rel_attn_bwd_ldp(int M, int L) { return (static_cast<size_t>(M) + L + 7) & ~size_t(7); }

txl_status launch_rel_attn_bwd(const AttnParams &p, const BwdParams &g, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_kv_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kKvLdsTotal)) != hipSuccess)
      return fail(TXL_ERR_HIP, "rel_attn_bwd: cannot raise the LDS limit to %zu bytes", kKvLdsTotal);
    attr_set = true;
  }
  if (p.kv_sl < DH || p.r_sl < DH || p.q_sl < DH || p.o_sl < DH || g.do_sl < DH)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: bf16 row strides must be >= d_h");
  const int64_t ML = static_cast<int64_t>(p.M) + p.L;
  if ((ML + KB2) * p.kv_sl * 2 >= (int64_t(1) << 31) || (ML + 2 * QT) * p.r_sl * 2 >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: key / R rows span more than 2 GiB per head");
  if ((static_cast<int64_t>(p.L) * g.ldp + 16) * 2 >= (int64_t(1) << 30))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: g rows span more than 1 GiB per (batch row, head)");
  const int B = p.B, H = p.H, L = p.L;
  const int64_t BHL = static_cast<int64_t>(B) * H * L;
  const int64_t blocks = (ML + KB2 - 1) / KB2 * B * H;
  if (blocks > 0x7fffffffLL || BHL * 8 / 256 + 1 > 0x7fffffffLL)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn_bwd: grid too large");
  (void)hipGetLastError();
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((BHL * 8 + 255) / 256)), dim3(256), 0, s,
                     p, g);
  txl_status st = check_launch("bwd_prep_kernel");
  if (st != TXL_OK) return st;
  const int n_kb = (static_cast<int>(ML) + KB2 - 1) / KB2;
  hipLaunchKernelGGL(bwd_kv_kernel, dim3(static_cast<unsigned>(static_cast<int64_t>(n_kb) * B * H)), dim3(256),
                     kKvLdsTotal, s, p, g, n_kb);
  if ((st = check_launch("bwd_kv_kernel")) != TXL_OK) return st;

  const int ml = static_cast<int>(ML);
  auto run = [&](BgParams q, int z_count) -> txl_status {
    q.valid = p.valid;
    q.M = p.M;
    q.L = L;
    const int64_t wgs = static_cast<int64_t>((q.rows + GT - 1) / GT) * z_count;
    hipLaunchKernelGGL(bgemm_kernel, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, s, q);
    return check_launch("bgemm_kernel");
  };
  const int64_t pz = static_cast<int64_t>(L) * g.ldp;      // g by key / by distance per (b, h)
  const int n_mt_q = (L + GT - 1) / GT;

  // dq = g K over keys, then + g R over distances, in one accumulator; the
  // column sums of the two shares give du and dv_bias
  BgParams q = {};
  q.rows = L; q.n_phase = 2;
  q.ph[0].kind = 1; q.ph[0].K = ml;
  q.ph[0].a = g.gm; q.ph[0].lda = g.ldp; q.ph[0].a_s1 = H * pz; q.ph[0].a_s2 = pz;
  q.ph[0].b = static_cast<const __bf16 *>(p.k); q.ph[0].ldb = p.kv_sl; q.ph[0].b_s1 = p.kv_sb;
  q.ph[0].b_s2 = p.kv_sh; q.ph[0].colsum = g.part_u;
  q.ph[1].kind = 2; q.ph[1].K = ml;
  q.ph[1].a = g.pm; q.ph[1].lda = g.ldp; q.ph[1].a_s1 = H * pz; q.ph[1].a_s2 = pz;
  q.ph[1].b = static_cast<const __bf16 *>(p.r); q.ph[1].ldb = p.r_sl; q.ph[1].b_s1 = 0;
  q.ph[1].b_s2 = p.r_sh; q.ph[1].colsum = g.part_v;
  if (g.rows.dq) {   // bf16 rows b*L + i, column h*64 + e
    q.c16 = g.rows.dq; q.ldc = g.rows.dq_ld; q.c_s1 = static_cast<int64_t>(L) * g.rows.dq_ld; q.c_s2 = DH;
  } else {
    q.c = g.dq; q.ldc = DH; q.c_s1 = static_cast<int64_t>(H) * L * DH; q.c_s2 = static_cast<int64_t>(L) * DH;
  }
  q.Z2 = H;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  // dR per batch row = sum over queries of g (q + v), by distance; summed over
  // batch rows by the reduction below
  q = BgParams{};
  q.rows = ml; q.n_phase = 1;
  q.ph[0].kind = 3; q.ph[0].K = L;
  q.ph[0].a = g.pm; q.ph[0].lda = g.ldp; q.ph[0].a_s1 = H * pz; q.ph[0].a_s2 = pz;
  q.ph[0].b = g.qv; q.ph[0].ldb = DH; q.ph[0].b_s1 = static_cast<int64_t>(H) * L * DH;
  q.ph[0].b_s2 = static_cast<int64_t>(L) * DH;
  q.c = g.part_r; q.ldc = DH; q.c_s1 = static_cast<int64_t>(H) * ml * DH; q.c_s2 = static_cast<int64_t>(ml) * DH;
  q.Z2 = H;
  if ((st = run(q, B * H)) != TXL_OK) return st;
  const int64_t n_r = static_cast<int64_t>(H) * ml * DH;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>(2 * H + (n_r + 255) / 256)), dim3(256), 0, s,
                     g.part_r, g.dr, n_r, g.part_u, g.part_v, g.du, g.dvb, B, H, n_mt_q, g.rows.dr,
                     g.rows.dr_ld, ml);
  return check_launch("bwd_reduce_kernel");
}

}  // namespace txl
