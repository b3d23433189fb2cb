// Relative-position table R = S W_R^T per head.
//
// [P1] "Transformer-XL" notes, "Dimension Walkthrough": R holds one row per
// relative distance, from the farthest memory slot down to distance 0, so
// row t holds distance M+L-1-t. [P4] "Transformer-XL" glossary: R is a
// sinusoidal embedding of the distance, projected per head. The sinusoid is
// the concatenated form S(delta, k) = sin(delta f_k) | cos(delta f_k),
// f_k = 10000^(-2k/d).
//
// R depends only on the weights and on (M, L), so it is built once per
// model; this kernel favours accuracy over speed: the sinusoid is evaluated
// in fp64 and held in LDS as fp32, the projection accumulates in fp32.
// One workgroup covers kRows distances; each thread owns output columns and
// streams its W_R row once for all kRows distances.
#include <hip/hip_runtime.h>

#include <cmath>

#include "txl_internal.h"

namespace txl {
namespace {

constexpr int kRows = 4;
constexpr int kThreads = 256;

__device__ inline float load_f(const float *p) { return *p; }
__device__ inline float load_f(const __bf16 *p) { return static_cast<float>(*p); }
__device__ inline void store_f(float *p, float x) { *p = x; }
__device__ inline void store_f(__bf16 *p, float x) { *p = static_cast<__bf16>(x); }

template <typename T>
__global__ __launch_bounds__(kThreads) void rel_pos_table_kernel(
    int ML, int d, int HD, const T *__restrict__ w, T *__restrict__ r) {
  extern __shared__ float s_emb[];  // [kRows][d]
  const int t0 = blockIdx.x * kRows;
  const int half = d / 2;
  for (int e = threadIdx.x; e < kRows * d; e += kThreads) {
    const int rr = e / d, k = e - rr * d;
    const int t = t0 + rr;
    float val = 0.0f;
    if (t < ML) {
      const double dist = static_cast<double>(ML - 1 - t);
      const int kk = k < half ? k : k - half;
      const double f = pow(10000.0, -2.0 * kk / static_cast<double>(d));
      const double ang = dist * f;
      val = static_cast<float>(k < half ? sin(ang) : cos(ang));
    }
    s_emb[e] = val;
  }
  __syncthreads();
  for (int o = threadIdx.x; o < HD; o += kThreads) {
    float acc[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) acc[rr] = 0.0f;
    const T *wrow = w + static_cast<int64_t>(o) * d;
    for (int k = 0; k < d; ++k) {
      const float wv = load_f(wrow + k);
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) acc[rr] += s_emb[rr * d + k] * wv;
    }
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
      const int t = t0 + rr;
      if (t < ML) store_f(r + static_cast<int64_t>(t) * HD + o, acc[rr]);
    }
  }
}

}  // namespace

txl_status launch_rel_pos_table(txl_dtype dt, int M, int L, int d, int HD,
                                const void *w_r, void *r, hipStream_t s) {
  const int ML = M + L;
  const size_t lds = static_cast<size_t>(kRows) * d * sizeof(float);
  if (lds > 64 * 1024) return fail(TXL_ERR_UNSUPPORTED, "rel_pos_table: d = %d too large", d);
  const dim3 grid((ML + kRows - 1) / kRows);
  (void)hipGetLastError();
  if (dt == TXL_F32)
    hipLaunchKernelGGL(rel_pos_table_kernel<float>, grid, dim3(kThreads), lds, s, ML, d, HD,
                       static_cast<const float *>(w_r), static_cast<float *>(r));
  else
    hipLaunchKernelGGL(rel_pos_table_kernel<__bf16>, grid, dim3(kThreads), lds, s, ML, d, HD,
                       static_cast<const __bf16 *>(w_r), static_cast<__bf16 *>(r));
  return check_launch("rel_pos_table_kernel");
}

}  // namespace txl
