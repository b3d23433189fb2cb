// Relative-position table R = S W_R^T per head.
//
// [P1] "Transformer-XL" notes, "Dimension Walkthrough": R holds one row per
// relative distance, from the farthest memory slot down to distance 0, so
// row t holds distance M+L-1-t. [P4] "Transformer-XL" glossary: R is a
// sinusoidal embedding of the distance, projected per head. The sinusoid is
// the concatenated form S(delta, k) = sin(delta f_k) | cos(delta f_k),
// f_k = 10000^(-2k/d).
//
// A register-tiled fp32 product: one workgroup computes 32 distances x 64
// output columns, each thread 2 x 4 of them, over slabs of 32 of the d
// sinusoid dimensions. The sinusoid slab is evaluated in place: the
// frequencies once per workgroup in fp64 (in turns, f_k / 2pi), each angle
// delta*f_k/2pi in fp64 reduced to its fractional part in fp64, then the
// hardware sin / cos of that fraction of a turn in fp32, so an entry is
// accurate to about 1e-6 for any distance. W_R slabs of 64 dims go through
// LDS, loaded as 16-byte chunks (consecutive threads along a row) one slab
// ahead into registers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "txl_internal.h"

namespace txl {
namespace {

constexpr int TT = 32;        // distances per workgroup
constexpr int TO = 64;        // output columns per workgroup
constexpr int TK = 64;        // sinusoid dimensions per slab
constexpr int kThreads = 256; // 16 x 16 threads, each 2 distances x 4 columns
constexpr int kMaxHalf = 2048;  // d <= 4096

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void store_f(float *p, float x) { *p = x; }
__device__ inline void store_f(__bf16 *p, float x) { *p = static_cast<__bf16>(x); }

// The W_R slab [TO columns][TK dims] in registers: one 16-byte chunk per
// thread for bf16 (8 dims), two for fp32 (4 dims each); chunks of rows past
// HD or dims past d read as zero.
template <typename T>
struct WSlab {
  static constexpr int kPer = 16 / sizeof(T);                   // elements per chunk
  static constexpr int kChunks = TO * TK / kPer / kThreads;     // chunks per thread
  u32x4 v[kChunks];
  // vec: rows start 16-byte aligned (w aligned, d * sizeof(T) a multiple of 16)
  __device__ void load(const T *w, int d, int HD, int o0, int k0, int tid, bool vec) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int e = tid + c * kThreads;
      const int oo = e / (TK / kPer), kc = e % (TK / kPer);
      const int o = o0 + oo, k = k0 + kc * kPer;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (vec && o < HD && k + kPer <= d) {
        z = *reinterpret_cast<const u32x4 *>(w + static_cast<int64_t>(o) * d + k);
      } else if (o < HD && k < d) {  // unaligned rows or a row's ragged end
        T tmp[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          tmp[q] = k + q < d ? w[static_cast<int64_t>(o) * d + k + q] : static_cast<T>(0.0f);
        z = __builtin_bit_cast(u32x4, tmp);
      }
      v[c] = z;
    }
  }
  __device__ void store(float (*s_w)[TO + 4], int tid) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int e = tid + c * kThreads;
      const int oo = e / (TK / kPer), kc = e % (TK / kPer);
      const T *x = reinterpret_cast<const T *>(&v[c]);
#pragma unroll
      for (int q = 0; q < kPer; ++q) s_w[kc * kPer + q][oo] = static_cast<float>(x[q]);
    }
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rel_pos_table_kernel(
    int ML, int d, int HD, const T *__restrict__ w, T *__restrict__ r, bool vec) {
  __shared__ double s_f[kMaxHalf];          // f_k / 2pi for k < d/2
  __shared__ float s_s[TK][TT + 4];          // sinusoid slab, [k][distance]
  __shared__ float s_w[TK][TO + 4];          // W_R slab, [k][output column]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TT, o0 = blockIdx.y * TO;
  const int half = d / 2;
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  for (int k = tid; k < half; k += kThreads)
    s_f[k] = pow(10000.0, -2.0 * k / static_cast<double>(d)) * kInvTwoPi;
  const int tx = tid & 15, ty = tid >> 4;   // columns 4tx..4tx+3, distances 2ty, 2ty+1
  float acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  WSlab<T> nxt;
  nxt.load(w, d, HD, o0, 0, tid, vec);
  __syncthreads();
  for (int k0 = 0; k0 < d; k0 += TK) {
    nxt.store(s_w, tid);
    if (k0 + TK < d) nxt.load(w, d, HD, o0, k0 + TK, tid, vec);  // in flight during this slab
    for (int e = tid; e < TT * TK; e += kThreads) {
      const int tt = e % TT, kk = e / TT;
      const int t = t0 + tt, k = k0 + kk;
      float val = 0.0f;
      if (t < ML && k < d) {
        const bool is_sin = k < half;
        const double rev = static_cast<double>(ML - 1 - t) * s_f[is_sin ? k : k - half];
        const float frac = static_cast<float>(rev - rint(rev));  // in [-1/2, 1/2] turn
        val = is_sin ? __builtin_amdgcn_sinf(frac) : __builtin_amdgcn_cosf(frac);
      }
      s_s[kk][tt] = val;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < TK; ++kk) {
      const float a0 = s_s[kk][2 * ty], a1 = s_s[kk][2 * ty + 1];
      float b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = s_w[kk][4 * tx + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[0][j] += a0 * b[j];
        acc[1][j] += a1 * b[j];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 2 * ty + i;
    if (t >= ML) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = o0 + 4 * tx + j;
      if (o < HD) store_f(r + static_cast<int64_t>(t) * HD + o, acc[i][j]);
    }
  }
}

// The sinusoid rows, for the gradient of W_R: st[t, k] = S(M+L-1-t, k) in
// bf16 (the same evaluation as the table above).
__global__ __launch_bounds__(kThreads) void sinusoid_rows_kernel(int ML, int d,
                                                                 __bf16 *__restrict__ st) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= static_cast<int64_t>(ML) * d) return;
  const int t = static_cast<int>(e / d), k = static_cast<int>(e - static_cast<int64_t>(t) * d);
  const int half = d / 2;
  const bool is_sin = k < half;
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  const double f = pow(10000.0, -2.0 * (is_sin ? k : k - half) / static_cast<double>(d)) * kInvTwoPi;
  const double rev = static_cast<double>(ML - 1 - t) * f;
  const float frac = static_cast<float>(rev - rint(rev));
  st[e] = static_cast<__bf16>(is_sin ? __builtin_amdgcn_sinf(frac) : __builtin_amdgcn_cosf(frac));
}

}  // namespace

txl_status launch_sinusoid_rows(int M, int L, int d, void *st, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(M + L) * d;
  if (total == 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sinusoid_rows_kernel, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, M + L, d, static_cast<__bf16 *>(st));
  return check_launch("sinusoid_rows_kernel");
}

txl_status launch_rel_pos_table(txl_dtype dt, int M, int L, int d, int HD,
                                const void *w_r, void *r, hipStream_t s) {
  const int ML = M + L;
  if (d / 2 > kMaxHalf) return fail(TXL_ERR_UNSUPPORTED, "rel_pos_table: d = %d too large", d);
  const dim3 grid((ML + TT - 1) / TT, (HD + TO - 1) / TO);
  const size_t es = dt == TXL_F32 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(w_r) % 16 == 0) && (static_cast<size_t>(d) * es) % 16 == 0;
  (void)hipGetLastError();
  if (dt == TXL_F32)
    hipLaunchKernelGGL(rel_pos_table_kernel<float>, grid, dim3(kThreads), 0, s, ML, d, HD,
                       static_cast<const float *>(w_r), static_cast<float *>(r), vec);
  else
    hipLaunchKernelGGL(rel_pos_table_kernel<__bf16>, grid, dim3(kThreads), 0, s, ML, d, HD,
                       static_cast<const __bf16 *>(w_r), static_cast<__bf16 *>(r), vec);
  return check_launch("rel_pos_table_kernel");
}

}  // namespace txl
