// Kernels of the stack's segment gradients (the products run on gemm.hip and
// dw_gemm.hip): the batched weight transposes of the input-gradient
// products, the [memory; segment] rows as one matrix, deterministic sums of
// split-K partials, the LayerNorm backward and the embedding scatter.
//
// [P1] "Transformer-XL" notes, "Why Stop Gradient" and "Training Loop
// Sketch"; [P2] "019 Transformer-XL", section "stop-gradient到底切断哪里":
// the memory is a constant of the segment's graph, so none of these kernels
// produces a gradient for it; its rows still enter the W^K / W^V products.
// Every reduction runs in a fixed order, so the gradients are bit-for-bit
// reproducible.
#include <hip/hip_runtime.h>

#include <cmath>

#include "txl_internal.h"

namespace txl {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;  // transpose tile

// Up to kMaxTransposes bf16 transposes in one launch, y[c, col0 + q] =
// x[q, c], R and C multiples of 64: workgroup t takes 64 x 64 tile t of the
// job whose tile range holds it. Each thread loads two 16-byte row chunks
// of the tile into LDS and stores two 16-byte chunks of the transposed
// tile, eight rows of one column gathered from LDS.
struct TransposeBatch {
  TransposeJob job[kMaxTransposes];
  int tile0[kMaxTransposes + 1];  // job k owns tiles [tile0[k], tile0[k + 1])
  int n;
};

__global__ __launch_bounds__(256) void transpose_batch_kernel(TransposeBatch tb) {
  __shared__ __bf16 tile[kT][kT + 2];
  int k = 0;
  while (k + 1 < tb.n && static_cast<int>(blockIdx.x) >= tb.tile0[k + 1]) ++k;
  const TransposeJob &jb = tb.job[k];
  const int t = blockIdx.x - tb.tile0[k];
  const int n_tc = jb.C / kT;
  const int q0 = (t / n_tc) * kT, c0 = (t % n_tc) * kT;
  const int tid = threadIdx.x;
  const __bf16 *x = static_cast<const __bf16 *>(jb.x);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 3) + 32 * i, ch = tid & 7;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(q0 + row) * jb.ldx + c0 + 8 * ch);
    const __bf16 *e = reinterpret_cast<const __bf16 *>(&v);
#pragma unroll
    for (int m = 0; m < 8; ++m) tile[row][8 * ch + m] = e[m];
  }
  __syncthreads();
  __bf16 *y = static_cast<__bf16 *>(jb.y);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cc = (tid >> 3) + 32 * i, qc = tid & 7;
    __bf16 e[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) e[m] = tile[8 * qc + m][cc];
    *reinterpret_cast<u32x4 *>(y + static_cast<int64_t>(c0 + cc) * jb.ldy + jb.col0 + q0 + 8 * qc) =
        __builtin_bit_cast(u32x4, e);
  }
}

// [memory; segment] rows of every batch row as one matrix, y [B*(M+L), d]:
// row b*(M+L) + j is memory row j of batch row b (logical order) when j < M
// and the row holds it (j >= M - valid[b]), zero for a slot it does not
// hold, and segment row j - M otherwise. 16-byte chunks.
__global__ __launch_bounds__(256) void gather_ext_kernel(const u32x4 *__restrict__ mem,
                                                         const int32_t *__restrict__ valid,
                                                         const u32x4 *__restrict__ seg, int B, int M,
                                                         int L, int cpr, u32x4 *__restrict__ y) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(B) * (M + L) * cpr;
  if (e >= total) return;
  const int64_t row = e / cpr;
  const int c = static_cast<int>(e - row * cpr);
  const int b = static_cast<int>(row / (M + L)), j = static_cast<int>(row - static_cast<int64_t>(b) * (M + L));
  u32x4 v = {0u, 0u, 0u, 0u};
  if (j >= M) {
    v = seg[(static_cast<int64_t>(b) * L + (j - M)) * cpr + c];
  } else {
    const int vl = min(max(valid[b], 0), M);
    if (j >= M - vl) v = mem[(static_cast<int64_t>(b) * M + j) * cpr + c];
  }
  y[e] = v;
}

// Column sums of many parts over few columns, for up to four part sets in
// one launch (the LayerNorm gamma and beta partials of a layer's two
// LayerNorms: hundreds of parts, d columns): blockIdx.y picks the set, a
// workgroup owns 8 columns, its 32 thread groups each add every 32nd part in
// order, and the 32 group sums are added in group order.
constexpr int kColGroups = 32, kColsPerBlock = 8, kMaxColSets = 4;
struct ColSets {
  const float *part[kMaxColSets];
  float *out[kMaxColSets];
};
__global__ __launch_bounds__(256) void reduce_cols_kernel(ColSets cs, int S, int64_t stride, int64_t n) {
  __shared__ float red[kColGroups][kColsPerBlock];
  const float *part = cs.part[0];
  float *out = cs.out[0];
#pragma unroll
  for (int k = 1; k < kMaxColSets; ++k)
    if (static_cast<int>(blockIdx.y) == k) {
      part = cs.part[k];
      out = cs.out[k];
    }
  const int cl = threadIdx.x % kColsPerBlock, grp = threadIdx.x / kColsPerBlock;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kColsPerBlock + cl;
  float acc = 0.0f;
  if (col < n) {
#pragma unroll 8
    for (int s = grp; s < S; s += kColGroups) acc += part[s * stride + col];
  }
  red[grp][cl] = acc;
  __syncthreads();
  if (grp == 0 && col < n) {
    float t = red[0][cl];
#pragma unroll
    for (int gq = 1; gq < kColGroups; ++gq) t += red[gq][cl];
    out[col] = t;
  }
}

// LayerNorm backward, one wave per row, rows [blockIdx.x * rpb, ...) per
// workgroup: dx = r (gdy - mean(gdy) - xhat mean(gdy xhat)), gdy = dy gamma,
// xhat = (x - mean) r; dx in fp32 and, when dxb is set, bf16. The gamma and
// beta gradients of the workgroup's rows (sum of dy xhat and of dy, rows in
// order within a wave, the four waves added in order) go to
// part_g / part_b [blockIdx.x, d].
constexpr int kLnMaxChunks = 16;  // d <= 4096
template <int NCH>
__global__ __launch_bounds__(256) void ln_backward_kernel(
    const float *__restrict__ x, const __bf16 *__restrict__ gamma, const float *__restrict__ dy,
    float *__restrict__ dx, __bf16 *__restrict__ dxb, float *__restrict__ part_g,
    float *__restrict__ part_b, int rows, int d, int rpb, float eps) {
  constexpr int MAXC = NCH > 0 ? NCH : kLnMaxChunks;
  constexpr int RC = MAXC < 8 ? MAXC : 8;  // chunks per pass of the partial-sum exchange
  __shared__ float red[4][2][RC * 256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = NCH > 0 ? NCH : d / 256;
  f32x4 ag[MAXC], ab[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    ag[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    ab[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int r_lo = blockIdx.x * rpb, r_hi = min(rows, r_lo + rpb);
  bf16x4 gmv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nch) gmv[c] = *reinterpret_cast<const bf16x4 *>(gamma + 256 * c + 4 * lane);
  // x and dy of a wave's next row are loaded while its current row is
  // computed (the last row's "next" is the row itself again, a cache hit)
  f32x4 xn[MAXC], gn[MAXC];
  auto load_row = [&](int rw) {
    const float *xr = x + static_cast<int64_t>(rw) * d;
    const float *gr = dy + static_cast<int64_t>(rw) * d;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) {
        xn[c] = *reinterpret_cast<const f32x4 *>(xr + 256 * c + 4 * lane);
        gn[c] = *reinterpret_cast<const f32x4 *>(gr + 256 * c + 4 * lane);
      }
  };
  if (r_lo + wave < r_hi) load_row(r_lo + wave);
  for (int row = r_lo + wave; row < r_hi; row += 4) {
    f32x4 xv[MAXC], gv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) {
        xv[c] = xn[c];
        gv[c] = gn[c];
      }
    load_row(row + 4 < r_hi ? row + 4 : row);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) s += (xv[c][0] + xv[c][1]) + (xv[c][2] + xv[c][3]);
    s = wave_sum(s);
    const float mean = s / d;
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = xv[c][e] - mean;
          ss += t * t;
        }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / d + eps);
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) {
        const bf16x4 gm = gmv[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xh = (xv[c][e] - mean) * rs;
          ag[c][e] += gv[c][e] * xh;
          ab[c][e] += gv[c][e];
          const float gdy = gv[c][e] * static_cast<float>(gm[e]);
          xv[c][e] = xh;
          gv[c][e] = gdy;
          m1 += gdy;
          m2 += gdy * xh;
        }
      }
    m1 = wave_sum(m1);
    m2 = wave_sum(m2);
    m1 /= d;
    m2 /= d;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) {
        f32x4 o4;
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o4[e] = rs * (gv[c][e] - m1 - xv[c][e] * m2);
          ob[e] = static_cast<__bf16>(o4[e]);
        }
        const int64_t at = static_cast<int64_t>(row) * d + 256 * c + 4 * lane;
        *reinterpret_cast<f32x4 *>(dx + at) = o4;
        if (dxb) *reinterpret_cast<bf16x4 *>(dxb + at) = ob;
      }
  }
  // the four waves' partial sums, added in wave order, RC chunks per pass
  for (int base = 0; base < nch; base += RC) {
#pragma unroll
    for (int c = 0; c < RC; ++c)
      if (base + c < nch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          red[wave][0][(c * 64 + lane) * 4 + e] = ag[base + c][e];
          red[wave][1][(c * 64 + lane) * 4 + e] = ab[base + c][e];
        }
    __syncthreads();
    const int n = (nch - base < RC ? nch - base : RC) * 256;
    for (int i = threadIdx.x; i < n; i += 256) {
      const float g = ((red[0][0][i] + red[1][0][i]) + red[2][0][i]) + red[3][0][i];
      const float bb = ((red[0][1][i] + red[1][1][i]) + red[2][1][i]) + red[3][1][i];
      // LDS index i = (c * 64 + lane) * 4 + e  <->  column 256 c + 4 lane + e
      const int c = i / 256, rem = i - c * 256;
      const int col = 256 * (base + c) + rem;
      part_g[static_cast<int64_t>(blockIdx.x) * d + col] = g;
      part_b[static_cast<int64_t>(blockIdx.x) * d + col] = bb;
    }
    __syncthreads();
  }
}

// demb[v, :] = sum of dh0[p, :] over the positions p with tokens[p] == v, in
// position order (rows of v with no token are 0; ids outside [0, vocab) add
// nothing). A workgroup owns 32 vocabulary rows and 256 columns: every wave
// scans the tokens 64 at a time with one ballot, and the matches are added
// to an LDS accumulator in position order. The tokens of eight such rounds
// are loaded together (clamped to the last position, so the loads need no
// branch): a scan that loaded one round at a time waited a memory round trip
// per 64 tokens.
constexpr int kEmbRows = 32, kEmbRounds = 8;
__global__ __launch_bounds__(256) void embed_backward_kernel(const int32_t *__restrict__ tokens,
                                                             int n_tok, const float *__restrict__ dh0,
                                                             int d, int vocab,
                                                             float *__restrict__ demb) {
  __shared__ float acc[kEmbRows][256];
  const int v0 = blockIdx.x * kEmbRows, c0 = blockIdx.y * 256;
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = c0 + tid;
#pragma unroll
  for (int r = 0; r < kEmbRows; ++r) acc[r][tid] = 0.0f;
  for (int pb = 0; pb < n_tok; pb += 64 * kEmbRounds) {
    int tv[kEmbRounds];
#pragma unroll
    for (int s = 0; s < kEmbRounds; ++s) {
      const int p = pb + 64 * s + lane;
      tv[s] = tokens[p < n_tok ? p : n_tok - 1];
    }
#pragma unroll
    for (int s = 0; s < kEmbRounds; ++s) {
      const int p0 = pb + 64 * s;
      const int t = p0 + lane < n_tok ? tv[s] : -1;
      uint64_t hit = __builtin_amdgcn_ballot_w64(t >= v0 && t < v0 + kEmbRows && t < vocab);
      while (hit) {                     // the same mask in every wave: uniform
        const int k = __builtin_ctzll(hit);
        hit &= hit - 1;
        const int tk = __shfl(t, k);
        if (col < d) acc[tk - v0][tid] += dh0[static_cast<int64_t>(p0 + k) * d + col];
      }
    }
  }
  if (col >= d) return;
#pragma unroll 4
  for (int r = 0; r < kEmbRows; ++r)
    if (v0 + r < vocab) demb[static_cast<int64_t>(v0 + r) * d + col] = acc[r][tid];
}

__global__ void copy_i32_kernel(const int32_t *__restrict__ src, int32_t *__restrict__ dst, int n) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) dst[e] = src[e];
}

}  // namespace

txl_status launch_transpose_batch(const TransposeJob *jobs, int n, hipStream_t s) {
  if (n < 1 || n > kMaxTransposes) return fail(TXL_ERR_INVALID_ARG, "transpose_batch: %d jobs", n);
  TransposeBatch tb = {};
  tb.n = n;
  int64_t tiles = 0;
  for (int k = 0; k < n; ++k) {
    const TransposeJob &j = jobs[k];
    if (j.R <= 0 || j.C <= 0 || j.R % kT || j.C % kT || j.ldx % 8 || j.ldy % 8 || j.col0 % 8 ||
        j.ldx < j.C || j.ldy < j.col0 + j.R || reinterpret_cast<uintptr_t>(j.x) % 16 ||
        reinterpret_cast<uintptr_t>(j.y) % 16)
      return fail(TXL_ERR_UNSUPPORTED, "transpose_batch: job %d shape or alignment", k);
    tb.job[k] = j;
    tb.tile0[k] = static_cast<int>(tiles);
    tiles += static_cast<int64_t>(j.R / kT) * (j.C / kT);
    if (tiles > 0x7fffffff) return fail(TXL_ERR_UNSUPPORTED, "transpose_batch: too many tiles");
  }
  tb.tile0[n] = static_cast<int>(tiles);
  (void)hipGetLastError();
  hipLaunchKernelGGL(transpose_batch_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, tb);
  return check_launch("transpose_batch_kernel");
}

txl_status launch_gather_ext(const void *mem, const int32_t *valid, const void *seg, int B, int M, int L,
                             int d, void *y, hipStream_t s) {
  if (d % 8) return fail(TXL_ERR_UNSUPPORTED, "gather_ext: d must be a multiple of 8");
  const int cpr = d / 8;
  const int64_t total = static_cast<int64_t>(B) * (M + L) * cpr;
  if (total == 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(gather_ext_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const u32x4 *>(mem), valid, static_cast<const u32x4 *>(seg), B, M, L, cpr,
                     static_cast<u32x4 *>(y));
  return check_launch("gather_ext_kernel");
}

txl_status launch_reduce_cols(const float *const *parts, float *const *outs, int n_sets, int S,
                              int64_t stride, int64_t n, hipStream_t s) {
  if (n == 0 || n_sets == 0) return TXL_OK;
  if (n_sets < 0 || n_sets > kMaxColSets)
    return fail(TXL_ERR_INVALID_ARG, "reduce_cols: %d part sets (at most %d)", n_sets, kMaxColSets);
  ColSets cs = {};
  for (int k = 0; k < n_sets; ++k) {
    cs.part[k] = parts[k];
    cs.out[k] = outs[k];
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL(reduce_cols_kernel,
                     dim3(static_cast<unsigned>((n + kColsPerBlock - 1) / kColsPerBlock), n_sets), dim3(256), 0,
                     s, cs, S, stride, n);
  return check_launch("reduce_cols_kernel");
}

// rows per workgroup of the LayerNorm backward: at least kLnBwdMinRows, about
// kLnBwdBlocks workgroups
constexpr int kLnBwdBlocks = 512, kLnBwdMinRows = 8;
int ln_backward_blocks(int rows, int *rpb) {
  *rpb = (rows + kLnBwdBlocks - 1) / kLnBwdBlocks;
  if (*rpb < kLnBwdMinRows) *rpb = kLnBwdMinRows;
  return (rows + *rpb - 1) / *rpb;
}

txl_status launch_ln_backward(const float *x, const void *gamma, const float *dy, float *dx,
                              void *dxb, float *part_g, float *part_b, int rows, int d, float eps,
                              hipStream_t s) {
  if (rows == 0) return TXL_OK;
  if (d % 256 || d > 4096) return fail(TXL_ERR_UNSUPPORTED, "ln_backward: d must be a multiple of 256, <= 4096");
  int rpb;
  const int blocks = ln_backward_blocks(rows, &rpb);
  (void)hipGetLastError();
  const __bf16 *g = static_cast<const __bf16 *>(gamma);
  __bf16 *xb = static_cast<__bf16 *>(dxb);
  switch (d / 256) {
    case 1: hipLaunchKernelGGL(ln_backward_kernel<1>, dim3(blocks), dim3(256), 0, s, x, g, dy, dx, xb, part_g, part_b, rows, d, rpb, eps); break;
    case 2: hipLaunchKernelGGL(ln_backward_kernel<2>, dim3(blocks), dim3(256), 0, s, x, g, dy, dx, xb, part_g, part_b, rows, d, rpb, eps); break;
    case 3: hipLaunchKernelGGL(ln_backward_kernel<3>, dim3(blocks), dim3(256), 0, s, x, g, dy, dx, xb, part_g, part_b, rows, d, rpb, eps); break;
    case 4: hipLaunchKernelGGL(ln_backward_kernel<4>, dim3(blocks), dim3(256), 0, s, x, g, dy, dx, xb, part_g, part_b, rows, d, rpb, eps); break;
    default: hipLaunchKernelGGL(ln_backward_kernel<0>, dim3(blocks), dim3(256), 0, s, x, g, dy, dx, xb, part_g, part_b, rows, d, rpb, eps); break;
  }
  return check_launch("ln_backward_kernel");
}

txl_status launch_embed_backward(const int32_t *tokens, int n_tok, const float *dh0, int d,
                                 int vocab, float *demb, hipStream_t s) {
  const dim3 grid((vocab + kEmbRows - 1) / kEmbRows, (d + 255) / 256);
  (void)hipGetLastError();
  hipLaunchKernelGGL(embed_backward_kernel, grid, dim3(256), 0, s, tokens, n_tok, dh0, d, vocab, demb);
  return check_launch("embed_backward_kernel");
}

txl_status launch_copy_i32(const int32_t *src, int32_t *dst, int n, hipStream_t s) {
  if (n == 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return check_launch("copy_i32_kernel");
}

}  // namespace txl
