// Kernels of the stack's segment gradients (the layer GEMMs themselves run on
// the GEMM of gemm.hip): tiled transposes into bf16 GEMM operands, the
// packing of the attention's per-head gradients, deterministic sums of
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

constexpr int kT = 64;  // transpose tile

__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(__bf16 x) { return static_cast<float>(x); }

// y[c, col0 + q] = x_row(q)[c] for source rows q in [0, R) and 0 for
// R <= q < r_pad, columns c in [0, C). Source row q sits in group
// g = q / (g1 + g2) at j = q mod (g1 + g2): row g*g1 + j of x1 when j < g1,
// else row g*g2 + (j - g1) of x2, both with row stride ldx (a plain matrix
// is g1 = R, g2 = 0; [memory; segment] of every batch row is g1 = M,
// g2 = L). With valid1 set, x1 rows j < g1 - valid1[g] (memory slots a
// batch row does not hold) read as 0. 64 x 64 tiles through LDS, both sides
// coalesced.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ x1, int g1,
                                                        const int32_t *__restrict__ valid1,
                                                        const T *__restrict__ x2, int g2,
                                                        int64_t ldx, int R, int C, int r_pad,
                                                        __bf16 *__restrict__ y, int64_t ldy,
                                                        int col0) {
  __shared__ float tile[kT][kT + 1];
  const int c0 = blockIdx.x * kT, q0 = blockIdx.y * kT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int gs = g1 + g2;
#pragma unroll 4
  for (int k = 0; k < kT / 4; ++k) {
    const int qq = ty + 4 * k, q = q0 + qq, c = c0 + tx;
    float v = 0.0f;
    if (q < R && c < C) {
      const int g = q / gs, j = q - g * gs;
      bool held = true;
      if (j < g1 && valid1) {
        const int vl = min(max(valid1[g], 0), g1);
        held = j >= g1 - vl;
      }
      const T *row = j < g1 ? x1 + (static_cast<int64_t>(g) * g1 + j) * ldx
                            : x2 + (static_cast<int64_t>(g) * g2 + (j - g1)) * ldx;
      if (held) v = to_f(row[c]);
    }
    tile[qq][tx] = v;
  }
  __syncthreads();
#pragma unroll 4
  for (int k = 0; k < kT / 4; ++k) {
    const int cc = ty + 4 * k, c = c0 + cc, q = q0 + tx;
    if (c < C && q < r_pad) y[static_cast<int64_t>(c) * ldy + col0 + q] = static_cast<__bf16>(tile[tx][cc]);
  }
}

// Per-head fp32 gradients g [B, H, T, 64] (T keys or queries per batch row)
// into bf16 GEMM operands: the transposed merge yt[h*64 + e, b*T + j] (row
// stride ldt; columns from B*T on are left to the caller) and, when y2 is
// set, the merged rows of the last L entries of every batch row,
// y2[b*L + j - (T-L), col0 + h*64 + e] (row stride ld2).
__global__ __launch_bounds__(256) void head_grad_pack_kernel(const float *__restrict__ g, int B,
                                                             int H, int T, __bf16 *__restrict__ yt,
                                                             int64_t ldt, __bf16 *__restrict__ y2,
                                                             int L, int64_t ld2, int col0) {
  __shared__ float tile[kT][kT + 1];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int j0 = blockIdx.x * kT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const float *src = g + static_cast<int64_t>(bh) * T * 64;
#pragma unroll 4
  for (int k = 0; k < kT / 4; ++k) {
    const int jj = ty + 4 * k, j = j0 + jj;
    const float v = j < T ? src[static_cast<int64_t>(j) * 64 + tx] : 0.0f;
    tile[jj][tx] = v;
    if (y2 && j < T && j >= T - L)
      y2[(static_cast<int64_t>(b) * L + (j - (T - L))) * ld2 + col0 + h * 64 + tx] = static_cast<__bf16>(v);
  }
  __syncthreads();
#pragma unroll 4
  for (int k = 0; k < kT / 4; ++k) {
    const int e = ty + 4 * k, j = j0 + tx;
    if (j < T)
      yt[static_cast<int64_t>(h * 64 + e) * ldt + static_cast<int64_t>(b) * T + j] =
          static_cast<__bf16>(tile[tx][e]);
  }
}

// out[i] = sum_{s < S} part[s * stride + i], s ascending (4 floats a thread)
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float *__restrict__ part, int S,
                                                           int64_t stride, int64_t n4,
                                                           float *__restrict__ out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n4) return;
  f32x4 acc = reinterpret_cast<const f32x4 *>(part)[e];
  for (int s = 1; s < S; ++s) acc += reinterpret_cast<const f32x4 *>(part + s * stride)[e];
  reinterpret_cast<f32x4 *>(out)[e] = acc;
}

// The same sum for many parts over few columns (the LayerNorm parameter
// partials: hundreds of parts, d columns): a workgroup owns 16 columns, its
// 16 thread groups each add every 16th part in order, and the 16 group sums
// are added in group order.
constexpr int kColGroups = 16;
__global__ __launch_bounds__(256) void reduce_cols_kernel(const float *__restrict__ part, int S,
                                                          int64_t stride, int64_t n,
                                                          float *__restrict__ out) {
  __shared__ float red[kColGroups][16];
  const int cl = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 16 + cl;
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
__global__ __launch_bounds__(256) void ln_backward_kernel(
    const float *__restrict__ x, const __bf16 *__restrict__ gamma, const float *__restrict__ dy,
    float *__restrict__ dx, __bf16 *__restrict__ dxb, float *__restrict__ part_g,
    float *__restrict__ part_b, int rows, int d, int rpb, float eps) {
  __shared__ float red[4][2][8 * 256];  // 8 of the row's 256-column chunks per pass (64 KB)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = d / 256;
  f32x4 ag[kLnMaxChunks], ab[kLnMaxChunks];
#pragma unroll
  for (int c = 0; c < kLnMaxChunks; ++c) {
    ag[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    ab[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int r_lo = blockIdx.x * rpb, r_hi = min(rows, r_lo + rpb);
  for (int row = r_lo + wave; row < r_hi; row += 4) {
    const float *xr = x + static_cast<int64_t>(row) * d;
    const float *gr = dy + static_cast<int64_t>(row) * d;
    f32x4 xv[kLnMaxChunks], gv[kLnMaxChunks];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kLnMaxChunks; ++c)
      if (c < nch) {
        xv[c] = *reinterpret_cast<const f32x4 *>(xr + 256 * c + 4 * lane);
        s += (xv[c][0] + xv[c][1]) + (xv[c][2] + xv[c][3]);
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    const float mean = s / d;
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < kLnMaxChunks; ++c)
      if (c < nch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = xv[c][e] - mean;
          ss += t * t;
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float rs = 1.0f / sqrtf(ss / d + eps);
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int c = 0; c < kLnMaxChunks; ++c)
      if (c < nch) {
        const bf16x4 gm = *reinterpret_cast<const bf16x4 *>(gamma + 256 * c + 4 * lane);
        gv[c] = *reinterpret_cast<const f32x4 *>(gr + 256 * c + 4 * lane);
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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      m1 += __shfl_xor(m1, o);
      m2 += __shfl_xor(m2, o);
    }
    m1 /= d;
    m2 /= d;
#pragma unroll
    for (int c = 0; c < kLnMaxChunks; ++c)
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
  // the four waves' partial sums, added in wave order
  for (int half = 0; half < 2; ++half) {  // chunks [8 half, 8 half + 8): LDS holds half the row
    if (half * 8 >= nch) break;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (half * 8 + c < nch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          red[wave][0][(c * 64 + lane) * 4 + e] = ag[half * 8 + c][e];
          red[wave][1][(c * 64 + lane) * 4 + e] = ab[half * 8 + c][e];
        }
    __syncthreads();
    const int n = (nch - half * 8 < 8 ? nch - half * 8 : 8) * 256;
    for (int i = threadIdx.x; i < n; i += 256) {
      const float g = ((red[0][0][i] + red[1][0][i]) + red[2][0][i]) + red[3][0][i];
      const float bb = ((red[0][1][i] + red[1][1][i]) + red[2][1][i]) + red[3][1][i];
      // LDS index i = (c * 64 + lane) * 4 + e  <->  column 256 c + 4 lane + e
      const int c = i / 256, rem = i - c * 256;
      const int col = 256 * (half * 8 + c) + rem;
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
// to an LDS accumulator in position order.
constexpr int kEmbRows = 32;
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
  for (int p0 = 0; p0 < n_tok; p0 += 64) {
    const int p = p0 + lane;
    const int t = p < n_tok ? tokens[p] : -1;
    uint64_t hit = __builtin_amdgcn_ballot_w64(t >= v0 && t < v0 + kEmbRows && t < vocab);
    while (hit) {                       // the same mask in every wave: uniform
      const int k = __builtin_ctzll(hit);
      hit &= hit - 1;
      const int tk = __shfl(t, k);
      if (col < d) acc[tk - v0][tid] += dh0[static_cast<int64_t>(p0 + k) * d + col];
    }
  }
  if (col >= d) return;
#pragma unroll 4
  for (int r = 0; r < kEmbRows; ++r)
    if (v0 + r < vocab) demb[static_cast<int64_t>(v0 + r) * d + col] = acc[r][tid];
}

// y[r, c] = 0 for rows r < n_rows and columns c in [c_from, c_to) (row stride ldy)
__global__ __launch_bounds__(256) void zero_cols_kernel(__bf16 *__restrict__ y, int n_rows, int64_t ldy,
                                                        int c_from, int c_to) {
  const int w = c_to - c_from;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(n_rows) * w) return;
  const int64_t r = e / w;
  y[r * ldy + c_from + (e - r * w)] = static_cast<__bf16>(0.0f);
}

__global__ void copy_i32_kernel(const int32_t *__restrict__ src, int32_t *__restrict__ dst, int n) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) dst[e] = src[e];
}

}  // namespace

txl_status launch_transpose_bf16(const void *x1, int g1, const int32_t *valid1, const void *x2,
                                 int g2, int64_t ldx, bool src_f32, int R, int C, int r_pad,
                                 void *y, int64_t ldy, int col0, hipStream_t s) {
  if (C <= 0 || r_pad <= 0) return TXL_OK;
  if (g1 + g2 <= 0) return fail(TXL_ERR_INVALID_ARG, "transpose: empty row groups");
  const dim3 grid((C + kT - 1) / kT, (r_pad + kT - 1) / kT);
  (void)hipGetLastError();
  if (src_f32)
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float *>(x1), g1,
                       valid1, static_cast<const float *>(x2), g2, ldx, R, C, r_pad,
                       static_cast<__bf16 *>(y), ldy, col0);
  else
    hipLaunchKernelGGL(transpose_kernel<__bf16>, grid, dim3(256), 0, s, static_cast<const __bf16 *>(x1), g1,
                       valid1, static_cast<const __bf16 *>(x2), g2, ldx, R, C, r_pad,
                       static_cast<__bf16 *>(y), ldy, col0);
  return check_launch("transpose_kernel");
}

txl_status launch_head_grad_pack(const float *g, int B, int H, int T, void *yt, int64_t ldt,
                                 void *y2, int L, int64_t ld2, int col0, hipStream_t s) {
  if (B == 0 || T == 0) return TXL_OK;
  const dim3 grid((T + kT - 1) / kT, B * H);
  (void)hipGetLastError();
  hipLaunchKernelGGL(head_grad_pack_kernel, grid, dim3(256), 0, s, g, B, H, T, static_cast<__bf16 *>(yt), ldt,
                     static_cast<__bf16 *>(y2), L, ld2, col0);
  return check_launch("head_grad_pack_kernel");
}

txl_status launch_reduce_parts(const float *part, int S, int64_t stride, int64_t n, float *out,
                               hipStream_t s) {
  if (n == 0) return TXL_OK;
  (void)hipGetLastError();
  if (S > 16) {  // many parts: split them over thread groups
    hipLaunchKernelGGL(reduce_cols_kernel, dim3(static_cast<unsigned>((n + 15) / 16)), dim3(256), 0, s,
                       part, S, stride, n, out);
    return check_launch("reduce_cols_kernel");
  }
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s,
                     part, S, stride, n4, out);
  return check_launch("reduce_parts_kernel");
}

// rows per workgroup of the LayerNorm backward: at least 16, about 256 workgroups
int ln_backward_blocks(int rows, int *rpb) {
  *rpb = (rows + 255) / 256;
  if (*rpb < 16) *rpb = 16;
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
  hipLaunchKernelGGL(ln_backward_kernel, dim3(blocks), dim3(256), 0, s, x,
                     static_cast<const __bf16 *>(gamma), dy, dx, static_cast<__bf16 *>(dxb), part_g,
                     part_b, rows, d, rpb, eps);
  return check_launch("ln_backward_kernel");
}

txl_status launch_embed_backward(const int32_t *tokens, int n_tok, const float *dh0, int d,
                                 int vocab, float *demb, hipStream_t s) {
  const dim3 grid((vocab + kEmbRows - 1) / kEmbRows, (d + 255) / 256);
  (void)hipGetLastError();
  hipLaunchKernelGGL(embed_backward_kernel, grid, dim3(256), 0, s, tokens, n_tok, dh0, d, vocab, demb);
  return check_launch("embed_backward_kernel");
}

txl_status launch_zero_cols(void *y, int n_rows, int64_t ldy, int c_from, int c_to, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(n_rows) * (c_to - c_from);
  if (total <= 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(zero_cols_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<__bf16 *>(y), n_rows, ldy, c_from, c_to);
  return check_launch("zero_cols_kernel");
}

txl_status launch_copy_i32(const int32_t *src, int32_t *dst, int n, hipStream_t s) {
  if (n == 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return check_launch("copy_i32_kernel");
}

}  // namespace txl
