// Relative-position attention, VALU kernel: one thread per query row.
//
// Computes, for every visible key position j of query i,
//   A_ij = (q_i + u) . k_j + (q_i + v) . R_{i-j}
// ([P1] "Transformer-XL" notes, "Relative Positional Encoding", four terms
// regrouped as in [P3] section 2.2), then softmax(A * scale) over the visible
// keys and the weighted sum of v_j ([P1] "Dimension Walkthrough").
// Visible keys follow [P1] "Causal Mask With Memory": memory keys
// -valid_b <= j < 0 and current keys 0 <= j <= i.
//
// R_{i-j} is row t = j' + L - 1 - i of the table (j' = j + M is the logical
// key index): the shift is index arithmetic inside the tile, no padded copy.
//
// This kernel serves fp32 (exact fp32 arithmetic throughout); it is the
// simple, register-resident design: q+u, q+v and the output accumulator of a
// row live in one thread, key tiles of K, V and the R rows they need are
// staged in LDS, and the softmax is the streaming (online) form.
#include <hip/hip_runtime.h>

#include <cmath>

#include "txl_internal.h"

namespace txl {
namespace {

constexpr int DH = 64;             // head dimension served
constexpr int QT = 64;             // queries per workgroup (one per thread)
constexpr int KT = 32;             // keys per tile
constexpr int RT = KT + QT - 1;    // R rows one tile needs
constexpr int RP = DH + 1;         // padded R row: conflict-free skewed reads

__device__ inline float ld(const float *p) { return *p; }
__device__ inline void st(float *p, float x) { *p = x; }

template <typename T>
__global__ __launch_bounds__(QT) void rel_attn_valu_kernel(AttnParams p) {
  __shared__ float sk[KT][DH];
  __shared__ float sv[KT][DH];
  __shared__ float sr[RT][RP];

  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * QT;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int L = p.L, M = p.M;
  const int i = i0 + tid;
  const bool row_ok = i < L;
  int valid = p.valid ? p.valid[b] : M;
  valid = valid < 0 ? 0 : (valid > M ? M : valid);

  const T *q = static_cast<const T *>(p.q) + b * p.q_sb + h * p.q_sh;
  const T *k = static_cast<const T *>(p.k) + b * p.kv_sb + h * p.kv_sh;
  const T *v = static_cast<const T *>(p.v) + b * p.kv_sb + h * p.kv_sh;
  const T *r = static_cast<const T *>(p.r) + h * p.r_sh;
  const T *u = static_cast<const T *>(p.u) + h * DH;
  const T *vb = static_cast<const T *>(p.vb) + h * DH;

  float qu[DH], qv[DH], o[DH];
#pragma unroll
  for (int x = 0; x < DH; ++x) {
    const float qx = row_ok ? ld(q + static_cast<int64_t>(i) * p.q_sl + x) : 0.0f;
    qu[x] = qx + ld(u + x);
    qv[x] = qx + ld(vb + x);
    o[x] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  const int j_lo = M - valid;                      // first visible memory key
  const int i_last = (i0 + QT < L ? i0 + QT : L) - 1;
  const int j_end = M + i_last + 1;                // past the last key this block sees
  const int ML = M + L;

  for (int j0 = j_lo; j0 < j_end; j0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * DH; e += QT) {
      const int c = e / DH, x = e - c * DH;
      const int jj = j0 + c;
      const bool in = jj < j_end;
      sk[c][x] = in ? ld(k + static_cast<int64_t>(jj) * p.kv_sl + x) : 0.0f;
      sv[c][x] = in ? ld(v + static_cast<int64_t>(jj) * p.kv_sl + x) : 0.0f;
    }
    // rows t = j' + L - 1 - i for j' in the tile and i in the block
    const int t_base = j0 + L - i0 - QT;
    for (int e = tid; e < RT * DH; e += QT) {
      const int rr = e / DH, x = e - rr * DH;
      const int t = t_base + rr;
      sr[rr][x] = (t >= 0 && t < ML) ? ld(r + static_cast<int64_t>(t) * p.r_sl + x) : 0.0f;
    }
    __syncthreads();
    if (!row_ok) continue;

    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < KT; ++c) {
      const int jj = j0 + c;
      const int j = jj - M;
      const bool vis = j < 0 ? (j >= -valid) : (j <= i);
      float acc = 0.0f;
      if (vis) {
        const int rr = c + (QT - 1) - tid;  // = t - t_base
#pragma unroll
        for (int x = 0; x < DH; ++x) acc += qu[x] * sk[c][x] + qv[x] * sr[rr][x];
      }
      s[c] = vis ? acc * p.scale : -INFINITY;
      mt = fmaxf(mt, s[c]);
    }
    const float mn = fmaxf(m, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet for this row
    const float corr = expf(m - mn);  // m = -inf gives 0
    l *= corr;
#pragma unroll
    for (int x = 0; x < DH; ++x) o[x] *= corr;
#pragma unroll
    for (int c = 0; c < KT; ++c) {
      const float pc = expf(s[c] - mn);  // exp(-inf) = 0 for hidden keys
      l += pc;
#pragma unroll
      for (int x = 0; x < DH; ++x) o[x] += pc * sv[c][x];
    }
    m = mn;
  }

  if (!row_ok) return;
  const float inv = 1.0f / l;
  T *out = static_cast<T *>(p.out) + b * p.o_sb + h * p.o_sh + static_cast<int64_t>(i) * p.o_sl;
#pragma unroll
  for (int x = 0; x < DH; ++x) st(out + x, o[x] * inv);
  if (p.lse) p.lse[(static_cast<int64_t>(b) * p.H + h) * L + i] = m + logf(l);
}

}  // namespace

txl_status launch_rel_attn_valu(const AttnParams &p, txl_dtype dt,
                                hipStream_t s) {
  if (p.H > 65535 || p.B > 65535) return fail(TXL_ERR_UNSUPPORTED, "rel_attn: B or H > 65535");
  // fp32 only: bf16 attention always runs the MFMA kernel
  if (dt != TXL_F32) return fail(TXL_ERR_UNSUPPORTED, "rel_attn: the VALU kernel serves fp32 only");
  const dim3 grid((p.L + QT - 1) / QT, p.H, p.B);
  (void)hipGetLastError();
  hipLaunchKernelGGL(rel_attn_valu_kernel<float>, grid, dim3(QT), 0, s, p);
  return check_launch("rel_attn_valu_kernel");
}

}  // namespace txl
