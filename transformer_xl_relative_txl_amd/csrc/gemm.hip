// Dense layers of the stack: bf16 MFMA GEMM with fused epilogues, LayerNorm,
// embedding gather.
//
// [P1] "Transformer-XL" notes, "Segment-Level Recurrence": Q comes from the
// current segment, K and V from [SG(mem); H]; [P1] "Relation to KV Cache":
// the memory holds hidden states before projection, so each segment projects
// its memory again. The K/V GEMM therefore reads its A rows straight from the
// ring (in logical order, oldest first) and from the segment, never building
// [mem; H] in memory, and skips row tiles whose memory slots are all invalid.
//
// GEMM: C[m, n] = sum_k A[m, k] W[n, k] (W output-major, like a torch Linear
// weight), tiles of 128 or 64 rows x 128 or 64 columns per workgroup of 4
// waves (chosen per call so a launch has about two tiles per CU), blocks of
// v_mfma_f32_32x32x16_bf16, K in slabs of 64 (32 when K is not a multiple of
// 64) through two LDS buffers with one barrier per slab; global loads run two
// slabs ahead in two register sets.
// Tiles are handed out so that the tiles of one XCD are contiguous in
// row-major order (the hardware deals workgroups to the 8 XCDs round robin),
// which keeps a row tile's A rows in one L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "txl_internal.h"

namespace txl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// GELU with the exact erf form, erf by Abramowitz & Stegun formula 7.1.26
// (|error| <= 1.5e-7; about 5e-7 in fp32 arithmetic, far below the bf16
// rounding of the output): erf(|x|) = 1 - t (a1 + t (a2 + ... a5)) e^{-x^2},
// t = 1 / (1 + p |x|), odd in x. One reciprocal and one exp2 per element.
__device__ inline float gelu_erf(float v) {
  const float x = v * 0.7071067811865476f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  const float erf_x = copysignf(1.0f - poly * e, x);
  return 0.5f * v * (1.0f + erf_x);
}

// d/dv GELU(v) = Phi(v) + v phi(v), Phi from the same erf.
__device__ inline float gelu_erf_grad(float v) {
  const float x = v * 0.7071067811865476f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);  // exp(-v^2/2)
  const float erf_x = copysignf(1.0f - poly * e, x);
  return 0.5f * (1.0f + erf_x) + v * e * 0.3989422804014327f;
}

// Tile BM x BN (each 64 or 128) per workgroup of 4 waves arranged 2 x 2; a
// wave computes (BM/2) x (BN/2) as blocks of 32 x 32. K runs in slabs of BKS
// (32 or 64) through two LDS buffers: the next slab is loaded into registers while the
// MFMAs run and stored into the other buffer, one barrier per slab.
template <int E, int BM, int BN, int BKS>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams p) {
  constexpr int AS = BKS + 8;                    // LDS row stride (bf16 elements)
  constexpr int WM = BM / 64, WN = BN / 64;      // 32x32 blocks per wave
  constexpr int A_CH = BM * BKS / 8 / 256;       // 16-byte chunks per thread
  constexpr int B_CH = BN * BKS / 8 / 256;
  __shared__ __attribute__((aligned(16))) __bf16 sa[2][BM * AS];
  __shared__ __attribute__((aligned(16))) __bf16 sb[2][BN * AS];

  // XCD-contiguous tile assignment (a bijection on [0, T)); with split-K the
  // first T / k_splits indices are split 0, and so on
  const int T = gridDim.x;
  const int bid = blockIdx.x;
  const int x = bid % kXcds, local = bid / kXcds;
  const int q = T / kXcds, rem = T % kXcds;
  int tile = x * q + (x < rem ? x : rem) + local;
  int split = 0;
  if (E == kEpiPartialF32) {
    const int per = T / p.k_splits;
    split = tile / per;
    tile -= split * per;
  }
  const int n_tn = p.N / BN;
  const int tm = tile / n_tn, tn = tile - tm * n_tn;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  // this thread's A rows and W rows (16-byte chunk kc of each 32-wide slab)
  constexpr int CPR = BKS / 8;                   // 16-byte chunks per slab row
  constexpr int RPP = 256 / CPR;                 // rows covered per pass of the block
  const int kc = tid % CPR;
  const __bf16 *arow[A_CH];
  const __bf16 *wrow[B_CH];
  int any_valid = 0;
  // gather mode: the valid counts of the rows' batch rows are loaded first,
  // all at once (rows past the end read the last row's): loaded inside the
  // row logic, each was waited for on its own before the next
  int vrow[A_CH];
  if (p.gather) {
    const int ml = p.memM + p.segL;
#pragma unroll
    for (int j = 0; j < A_CH; ++j) {
      const int m = min(m0 + tid / CPR + RPP * j, p.rows - 1);
      vrow[j] = p.valid[m / ml];
    }
  }
#pragma unroll
  for (int j = 0; j < A_CH; ++j) {
    const int row = tid / CPR + RPP * j;
    const int m = m0 + row;
    const __bf16 *src = nullptr;
    if (m < p.rows) {
      if (!p.gather) {
        src = p.a + static_cast<int64_t>(m) * p.lda;
      } else {
        const int ml = p.memM + p.segL;
        const int b = m / ml, jl = m - b * ml;
        if (jl >= p.memM) {
          src = p.seg + (static_cast<int64_t>(b) * p.segL + (jl - p.memM)) * p.lda;
        } else {
          int valid = vrow[j];
          valid = valid < 0 ? 0 : (valid > p.memM ? p.memM : valid);
          if (jl >= p.memM - valid) {
            int64_t slot = p.head + jl;
            if (slot >= p.memM) slot -= p.memM;
            src = p.ring + (static_cast<int64_t>(b) * p.memM + slot) * p.lda;
          }
        }
      }
    }
    arow[j] = src;
    any_valid |= (src != nullptr);
  }
#pragma unroll
  for (int j = 0; j < B_CH; ++j) {
    const int n = n0 + tid / CPR + RPP * j;
    wrow[j] = n < p.n_split ? p.w0 + static_cast<int64_t>(n) * p.K
                            : p.w1 + static_cast<int64_t>(n - p.n_split) * p.K;
  }
  if (p.gather && !__syncthreads_or(any_valid)) return;  // all rows are empty memory slots

  // Every load is issued unconditionally, so the compiler counts the loads
  // in flight exactly and a slab's LDS store waits only for its own loads
  // (loads behind branches had made it wait for all of them, the prefetch
  // included): a row without data reads a W row instead and is zeroed when
  // stored.
  uint32_t a_ok = 0;
#pragma unroll
  for (int j = 0; j < A_CH; ++j) {
    if (arow[j]) a_ok |= 1u << j;
    else arow[j] = wrow[0];
  }

  // two register sets: slab ks+2 is loaded while slab ks is multiplied and
  // slab ks+1 waits in the other set for its LDS buffer
  u32x4 av[2][A_CH], wv[2][B_CH];
  auto load = [&](int set, int k0) {
#pragma unroll
    for (int j = 0; j < A_CH; ++j) av[set][j] = *reinterpret_cast<const u32x4 *>(arow[j] + k0 + 8 * kc);
#pragma unroll
    for (int j = 0; j < B_CH; ++j) wv[set][j] = *reinterpret_cast<const u32x4 *>(wrow[j] + k0 + 8 * kc);
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int j = 0; j < A_CH; ++j)
      *reinterpret_cast<u32x4 *>(&sa[buf][(tid / CPR + RPP * j) * AS + 8 * kc]) =
          (a_ok >> j) & 1u ? av[set][j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < B_CH; ++j)
      *reinterpret_cast<u32x4 *>(&sb[buf][(tid / CPR + RPP * j) * AS + 8 * kc]) = wv[set][j];
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < WN; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.0f;

  const int n_slab_all = p.K / BKS;
  const int ks0 = E == kEpiPartialF32 ? split * n_slab_all / p.k_splits : 0;
  const int ks1 = E == kEpiPartialF32 ? (split + 1) * n_slab_all / p.k_splits : n_slab_all;
  auto compute = [&](int cur) {
#pragma unroll
    for (int s = 0; s < BKS / 16; ++s) {
      bf16x8 af[WM], bfr[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        af[i] = *reinterpret_cast<const bf16x8 *>(
            &sa[cur][(wm * (BM / 2) + i * 32 + r) * AS + 16 * s + 8 * g]);
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
        bfr[jn] = *reinterpret_cast<const bf16x8 *>(
            &sb[cur][(wn * (BN / 2) + jn * 32 + r) * AS + 16 * s + 8 * g]);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma32(af[i], bfr[jn], acc[i][jn]);
    }
  };
  // slab ks lives in LDS buffer (ks - ks0) & 1 and register set (ks - ks0) & 1;
  // a buffer is refilled only after the barrier that ends its last readers
  // The loop runs while both of its loads are in range; the last one to
  // three slabs are peeled off with at most one more load.
  load(0, ks0 * BKS);
  load(1, min(ks0 + 1, ks1 - 1) * BKS);  // ks1 > ks0: every split holds a slab
  store(0, 0);
  __syncthreads();
  int ks = ks0;
  for (; ks + 3 < ks1; ks += 2) {
    load(0, (ks + 2) * BKS);
    compute(0);
    store(1, 1);
    __syncthreads();
    load(1, (ks + 3) * BKS);
    compute(1);
    store(0, 0);
    __syncthreads();
  }
  const int left = ks1 - ks;  // 1, 2 or 3 slabs: ks in buffer 0, ks + 1 in set 1
  if (left == 3) {
    load(0, (ks + 2) * BKS);
    compute(0);
    store(1, 1);
    __syncthreads();
    compute(1);
    store(0, 0);
    __syncthreads();
    compute(0);
  } else if (left == 2) {
    compute(0);
    store(1, 1);
    __syncthreads();
    compute(1);
  } else {
    compute(0);
  }
  __syncthreads();  // the epilogues reuse the LDS buffers

  // epilogue: register 4a+c of block (i, jn) holds
  // C[wm*BM/2 + 32i + 8a + 4g + c][wn*BN/2 + 32jn + r]
  if (E == kEpiLse) {
    // per column: this wave's rows (the two lane halves hold different rows
    // of the same column), then the two row halves of the tile through LDS
    float *xch = reinterpret_cast<float *>(&sa[0][0]);  // [BN][2]
    float wmx[WN], wsm[WN];
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      const int cl = wn * (BN / 2) + jn * 32 + r;
      const int n = n0 + cl;
      const int t = p.targets[n];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (x >> 2) + 4 * g + (x & 3);
          if (m < p.rows) mx = fmaxf(mx, acc[i][jn][x]);
          if (m == t) p.tgt[n] = acc[i][jn][x];  // the one lane holding (t, n)
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float sm = 0.0f;
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (x >> 2) + 4 * g + (x & 3);
          if (m < p.rows) sm += __builtin_amdgcn_exp2f((acc[i][jn][x] - mx) * 1.4426950408889634f);
        }
      sm += __shfl_xor(sm, 32);
      wmx[jn] = mx;
      wsm[jn] = sm;
      if (wm == 1 && g == 0) {
        xch[2 * cl] = mx;
        xch[2 * cl + 1] = sm;
      }
    }
    __syncthreads();
    if (wm == 0 && g == 0) {
#pragma unroll
      for (int jn = 0; jn < WN; ++jn) {
        const int cl = wn * (BN / 2) + jn * 32 + r;
        const float m1 = xch[2 * cl], s1 = xch[2 * cl + 1];
        const float mm = fmaxf(wmx[jn], m1);
        // a row half with no vocabulary rows has (-inf, 0)
        float ss = wsm[jn] * __builtin_amdgcn_exp2f((wmx[jn] - mm) * 1.4426950408889634f);
        if (s1 > 0.0f) ss += s1 * __builtin_amdgcn_exp2f((m1 - mm) * 1.4426950408889634f);
        const int64_t at = static_cast<int64_t>(tm) * p.N + n0 + cl;
        p.part_m[at] = mm;
        p.part_s[at] = ss;
      }
    }
    return;
  }
  const bool second = n0 >= p.n_split;
  // fp32-staged epilogue of the two GELU products that also touch a second
  // bf16 matrix of the output's shape (the stored pre-activation, or the
  // pre-activation the derivative is taken at): the tile goes to LDS as fp32
  // in two row halves (half a tile fits the A buffers) and every thread then
  // handles 8 consecutive columns of a row, with one 16-byte load of the
  // pre-activation and 16-byte stores, instead of one 2-byte access per
  // element. The arithmetic per element is the direct path's.
  constexpr bool kStagedF32 = BKS == 64 && (E == kEpiGeluGradBf16 || E == kEpiGeluBf16);
  if constexpr (kStagedF32) {
    const __bf16 *pre_in = E == kEpiGeluGradBf16 ? p.pre_in : nullptr;
    __bf16 *pre_out = E == kEpiGeluBf16 ? p.pre_out : nullptr;
    const uintptr_t al = reinterpret_cast<uintptr_t>(p.c0) | reinterpret_cast<uintptr_t>(p.c1) |
                         reinterpret_cast<uintptr_t>(pre_in) | reinterpret_cast<uintptr_t>(pre_out);
    if ((pre_in || pre_out) && (al & 15) == 0 && p.ldc % 8 == 0) {
      constexpr int HB = BM / 2;                 // rows per half (one wave row)
      constexpr int OSf = BN + 4;                // LDS row stride (floats)
      constexpr int CPR8 = BN / 8, RP8 = 256 / CPR8, IT8 = HB / RP8;
      static_assert(size_t(HB) * OSf * 4 <= sizeof(sa), "half a tile must fit the A buffers");
      static_assert(RP8 <= 32 && 32 % RP8 == 0, "row passes must tile 32-row blocks");
      float *ct = reinterpret_cast<float *>(&sa[0][0]);
      const int cc = tid % CPR8, rr0 = tid / CPR8;
      const int nc0 = (second ? n0 - p.n_split : n0) + cc * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // output row offsets of this thread's rows of the half (a 32-row
        // block never straddles an output segment: c_seg % 32 == 0), and the
        // pre-activation loaded before the barrier
        int64_t mo[IT8];
        bool ok[IT8];
        bf16x8 pin[IT8];
#pragma unroll
        for (int it = 0; it < IT8; ++it) {
          const int row = rr0 + RP8 * it;
          const int m = m0 + h * HB + row;
          ok[it] = m < p.rows;
          const int mb = m0 + h * HB + (RP8 * it / 32) * 32;
          mo[it] = (p.c_seg > 0 ? (mb / p.c_seg) * p.c_bstride + p.c_row0 + mb % p.c_seg
                                : static_cast<int64_t>(mb)) + (row & 31);
          if (E == kEpiGeluGradBf16)
            pin[it] = *reinterpret_cast<const bf16x8 *>(pre_in + (ok[it] ? mo[it] * p.ldc + nc0 : 0));
        }
        if (wm == h) {
#pragma unroll
          for (int jn = 0; jn < WN; ++jn)
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
              for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  const int row = i * 32 + 8 * a4 + 4 * g + c;
                  const int col = wn * (BN / 2) + jn * 32 + r;
                  ct[row * OSf + col] = acc[i][jn][4 * a4 + c];
                }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < IT8; ++it) {
          const int row = rr0 + RP8 * it;
          const f32x4 lo = *reinterpret_cast<const f32x4 *>(ct + row * OSf + cc * 8);
          const f32x4 hi = *reinterpret_cast<const f32x4 *>(ct + row * OSf + cc * 8 + 4);
          bf16x8 o, pre;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = e < 4 ? lo[e] : hi[e - 4];
            if (E == kEpiGeluBf16) {
              pre[e] = static_cast<__bf16>(v);
              v = gelu_erf(v);
            } else {
              v *= gelu_erf_grad(static_cast<float>(pin[it][e]));
            }
            o[e] = static_cast<__bf16>(v);
          }
          if (!ok[it]) continue;
          __bf16 *dst = static_cast<__bf16 *>(second ? p.c1 : p.c0) + mo[it] * p.ldc + nc0;
          *reinterpret_cast<bf16x8 *>(dst) = o;
          if (E == kEpiGeluBf16) *reinterpret_cast<bf16x8 *>(pre_out + mo[it] * p.ldc + nc0) = pre;
        }
        __syncthreads();  // the next half reuses the LDS rows
      }
      return;
    }
  }
  // Staged epilogue: the tile goes to LDS (free after the last barrier of the
  // loop) and leaves as 16-byte row chunks, the output row of each 32-row
  // block remapped once, instead of one 2-byte or 4-byte store per element.
  constexpr bool kStaged = BKS == 64 && (E == kEpiStoreBf16 || E == kEpiGeluBf16 ||
                                         ((E == kEpiResidualF32 || E == kEpiPartialF32) && BN == 64));
  // the pre-activation store takes the fp32-staged path above (or, unaligned,
  // the direct path)
  const bool direct_only = E == kEpiGeluBf16 && p.pre_out;
  if constexpr (kStaged) if (!direct_only) {
    typedef typename std::conditional<(E == kEpiStoreBf16 || E == kEpiGeluBf16), __bf16, float>::type OT;
    constexpr int VE = 16 / static_cast<int>(sizeof(OT));       // elements per 16-byte chunk
    constexpr int OS = BN + VE;                                  // LDS row stride (elements)
    constexpr int CPRo = BN / VE, RP = 256 / CPRo, IT = BM / RP;
    static_assert(size_t(BM) * OS * sizeof(OT) <= sizeof(sa), "staged tile must fit the A buffers");
    static_assert(32 % RP == 0 || RP % 32 == 0, "row passes must tile 32-row blocks");
    const uintptr_t al = reinterpret_cast<uintptr_t>(p.c0) | reinterpret_cast<uintptr_t>(p.c1);
    bool vec_ok = (al & 15) == 0 && p.ldc % VE == 0;
    if (E == kEpiResidualF32)
      vec_ok = vec_ok && p.ldres % 4 == 0 &&
               (p.res32 ? (reinterpret_cast<uintptr_t>(p.res32) & 15) == 0
                        : (reinterpret_cast<uintptr_t>(p.res) & 7) == 0);
    if (E == kEpiPartialF32) vec_ok = vec_ok && p.c_split_stride % 4 == 0;
    if (vec_ok) {
      OT *ct = reinterpret_cast<OT *>(&sa[0][0]);
      const int cc = tid % CPRo, rr0 = tid / CPRo;
      const int nc0 = (second ? n0 - p.n_split : n0) + cc * VE;
      // the residual of this thread's rows, loaded before the tile is staged
      // (rows past the end read row 0) and converted only where it is added
      constexpr int RI = E == kEpiResidualF32 ? IT : 1;
      f32x4 r32[RI];
      bf16x4 r16[RI];
      if constexpr (E == kEpiResidualF32) {
        if (p.res32) {
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int m = m0 + rr0 + RP * it;
            r32[it] = *reinterpret_cast<const f32x4 *>(p.res32 + static_cast<int64_t>(m < p.rows ? m : 0) * p.ldres + nc0);
          }
        } else {
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int m = m0 + rr0 + RP * it;
            r16[it] = *reinterpret_cast<const bf16x4 *>(p.res + static_cast<int64_t>(m < p.rows ? m : 0) * p.ldres + nc0);
          }
        }
      }
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int row = wm * (BM / 2) + i * 32 + 8 * a4 + 4 * g + c;
              const int col = wn * (BN / 2) + jn * 32 + r;
              float v = acc[i][jn][4 * a4 + c];
              if (E == kEpiGeluBf16) v = gelu_erf(v);
              ct[row * OS + col] = static_cast<OT>(v);
            }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int row = rr0 + RP * it;
        const int m = m0 + row;
        if (m >= p.rows) continue;
        // a 32-row block never straddles an output segment (c_seg % 32 == 0)
        const int mb = m0 + (RP * it / 32) * 32;
        const int64_t mo = (p.c_seg > 0 ? (mb / p.c_seg) * p.c_bstride + p.c_row0 + mb % p.c_seg
                                        : static_cast<int64_t>(mb)) + (row & 31);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ct + row * OS + cc * VE);
        if (E == kEpiPartialF32) {
          *reinterpret_cast<u32x4 *>(static_cast<float *>(p.c0) + split * p.c_split_stride + mo * p.ldc + nc0) = v;
        } else if (E == kEpiResidualF32) {
          f32x4 o = __builtin_bit_cast(f32x4, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] += p.res32 ? r32[RI > 1 ? it : 0][e] : static_cast<float>(r16[RI > 1 ? it : 0][e]);
          *reinterpret_cast<f32x4 *>(static_cast<float *>(second ? p.c1 : p.c0) + mo * p.ldc + nc0) = o;
        } else {
          *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(second ? p.c1 : p.c0) + mo * p.ldc + nc0) = v;
        }
      }
      return;
    }
  }
  // The residual and the stored pre-activation are loaded for all of the
  // lane's outputs before the first store, branch-free (rows past the end
  // read the first element): loaded one at a time, behind the row check and
  // after stores they might alias, each load was waited for on its own.
  constexpr bool kReads = E == kEpiResidualF32 || E == kEpiGeluGradBf16;
  float xin[kReads ? WN : 1][kReads ? WM : 1][kReads ? 16 : 1];
  if constexpr (kReads) {
    // element offset of output x of block (jn, i), or 0 past the last row
    auto at = [&](int jn, int i, int x) -> int64_t {
      const int nc = (second ? n0 - p.n_split : n0) + wn * (BN / 2) + jn * 32 + r;
      const int mb = m0 + wm * (BM / 2) + i * 32;
      const int mi = 8 * (x >> 2) + 4 * g + (x & 3);
      if (mb + mi >= p.rows) return 0;
      if (E == kEpiGeluGradBf16) {
        const int64_t ob = p.c_seg > 0 ? (mb / p.c_seg) * p.c_bstride + p.c_row0 + mb % p.c_seg
                                       : static_cast<int64_t>(mb);
        return (ob + mi) * p.ldc + nc;
      }
      return static_cast<int64_t>(mb + mi) * p.ldres + nc;
    };
    if (E == kEpiResidualF32 && p.res32) {
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int x = 0; x < 16; ++x) xin[jn][i][x] = p.res32[at(jn, i, x)];
    } else {
      const __bf16 *src = E == kEpiGeluGradBf16 ? p.pre_in : p.res;
      __bf16 raw[kReads ? WN : 1][kReads ? WM : 1][16];
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int x = 0; x < 16; ++x) raw[jn][i][x] = src[at(jn, i, x)];
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int x = 0; x < 16; ++x) xin[jn][i][x] = static_cast<float>(raw[jn][i][x]);
    }
  }
#pragma unroll
  for (int jn = 0; jn < WN; ++jn) {
    const int n = n0 + wn * (BN / 2) + jn * 32 + r;
    const int nc = second ? n - p.n_split : n;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      // a 32-row block never straddles an output segment (c_seg % 32 == 0)
      const int mb = m0 + wm * (BM / 2) + i * 32;
      const int64_t ob = p.c_seg > 0
                             ? (mb / p.c_seg) * p.c_bstride + p.c_row0 + mb % p.c_seg
                             : static_cast<int64_t>(mb);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int mi = 8 * a4 + 4 * g + c;
          const int m = mb + mi;
          if (m >= p.rows) continue;
          const int64_t mo = ob + mi;
          float v = acc[i][jn][4 * a4 + c];
          if (E == kEpiPartialF32) {
            static_cast<float *>(p.c0)[split * p.c_split_stride + mo * p.ldc + nc] = v;
          } else if (E == kEpiResidualF32) {
            v += xin[kReads ? jn : 0][kReads ? i : 0][kReads ? 4 * a4 + c : 0];
            static_cast<float *>(second ? p.c1 : p.c0)[mo * p.ldc + nc] = v;
          } else {
            if (E == kEpiGeluBf16) {
              if (p.pre_out) p.pre_out[mo * p.ldc + nc] = static_cast<__bf16>(v);
              v = gelu_erf(v);
            }
            if (E == kEpiGeluGradBf16) v *= gelu_erf_grad(xin[kReads ? jn : 0][kReads ? i : 0][kReads ? 4 * a4 + c : 0]);
            static_cast<__bf16 *>(second ? p.c1 : p.c0)[mo * p.ldc + nc] = static_cast<__bf16>(v);
          }
        }
    }
  }
}

// LayerNorm over rows of fp32 x: y = (x - mean) / sqrt(var + eps) * gamma + beta,
// biased variance, one wave per row, result rounded to bf16.
constexpr int kLnMaxChunks = 16;  // 4-float chunks per lane: d <= 4096

// NCH: 256-column chunks of a row when known at compile time (registers
// sized to the row), 0 for any d <= 4096.
template <int NP, int NCH>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *__restrict__ x,
                                                        int64_t part_stride,
                                                        const __bf16 *__restrict__ res,
                                                        const __bf16 *__restrict__ gamma,
                                                        const __bf16 *__restrict__ beta,
                                                        __bf16 *__restrict__ y, int rows, int d,
                                                        float eps, float *__restrict__ x_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  constexpr int MAXC = NCH > 0 ? NCH : kLnMaxChunks;
  const int nch = NCH > 0 ? NCH : d / 256;
  const float *xr = x + static_cast<int64_t>(row) * d;
  // every input of the row (x and its split-K partials, the residual, gamma
  // and beta) is loaded before any arithmetic: one memory round trip per row
  f32x4 v[MAXC], pv[MAXC][NP > 1 ? NP - 1 : 1];
  bf16x4 rr[MAXC], gm[MAXC], bt[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c < nch) {
      const int col = 256 * c + 4 * lane;
      v[c] = *reinterpret_cast<const f32x4 *>(xr + col);
#pragma unroll
      for (int part = 1; part < NP; ++part)
        pv[c][part - 1] = *reinterpret_cast<const f32x4 *>(xr + part * part_stride + col);
      if (res) rr[c] = *reinterpret_cast<const bf16x4 *>(res + static_cast<int64_t>(row) * d + col);
      gm[c] = *reinterpret_cast<const bf16x4 *>(gamma + col);
      bt[c] = *reinterpret_cast<const bf16x4 *>(beta + col);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c < nch) {
      // split-K partials in order, then the residual
#pragma unroll
      for (int part = 1; part < NP; ++part) v[c] += pv[c][part - 1];
      if (res) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[c][e] += static_cast<float>(rr[c][e]);
      }
      if (x_out) *reinterpret_cast<f32x4 *>(x_out + static_cast<int64_t>(row) * d + 256 * c + 4 * lane) = v[c];
      s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
    }
  }
  s = wave_sum(s);
  const float mean = s / d;
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = v[c][e] - mean;
        ss += t * t;
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / d + eps);
  __bf16 *yr = y + static_cast<int64_t>(row) * d;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c < nch) {
      const int col = 256 * c + 4 * lane;
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = static_cast<__bf16>((v[c][e] - mean) * inv * static_cast<float>(gm[c][e]) +
                                   static_cast<float>(bt[c][e]));
      *reinterpret_cast<bf16x4 *>(yr + col) = o;
    }
  }
}

// Combine the per-tile (max, sum of exponentials) of each token: a block of
// 256 threads covers 16 tokens, sixteen threads per token splitting the
// tiles (consecutive threads on consecutive tokens), then one combine in LDS.
constexpr int kFinTok = 16, kFinGrp = 16;
__global__ __launch_bounds__(256) void lse_finish_kernel(const float *__restrict__ part_m,
                                                         const float *__restrict__ part_s,
                                                         const float *__restrict__ tgt,
                                                         const int32_t *__restrict__ targets,
                                                         int n_tiles, int N, int vocab,
                                                         float *__restrict__ nll) {
  __shared__ float sm_m[kFinGrp][kFinTok], sm_s[kFinGrp][kFinTok];
  const int tl = threadIdx.x % kFinTok, grp = threadIdx.x / kFinTok;
  const int n = blockIdx.x * kFinTok + tl;
  float m = -INFINITY, s = 0.0f;
  if (n < N) {
    // four of the group's tiles loaded before the first is combined (tiles
    // past the end load the group's first and are skipped); the tiles are
    // combined in the same order as one at a time
    constexpr int kFinBatch = 4;
    for (int t0 = grp; t0 < n_tiles; t0 += kFinBatch * kFinGrp) {
      float mt[kFinBatch], st[kFinBatch];
#pragma unroll
      for (int u = 0; u < kFinBatch; ++u) {
        const int t = t0 + u * kFinGrp < n_tiles ? t0 + u * kFinGrp : t0;
        mt[u] = part_m[static_cast<int64_t>(t) * N + n];
        st[u] = part_s[static_cast<int64_t>(t) * N + n];
      }
#pragma unroll
      for (int u = 0; u < kFinBatch; ++u) {
        if (t0 + u * kFinGrp >= n_tiles || st[u] <= 0.0f) continue;
        if (mt[u] > m) {
          s = s * __expf(m - mt[u]) + st[u];
          m = mt[u];
        } else {
          s += st[u] * __expf(mt[u] - m);
        }
      }
    }
  }
  sm_m[grp][tl] = m;
  sm_s[grp][tl] = s;
  __syncthreads();
  if (grp != 0 || n >= N) return;
  float mm = sm_m[0][tl];
#pragma unroll
  for (int k = 1; k < kFinGrp; ++k) mm = fmaxf(mm, sm_m[k][tl]);
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < kFinGrp; ++k)
    if (sm_s[k][tl] > 0.0f) ss += sm_s[k][tl] * __expf(sm_m[k][tl] - mm);
  const int t = targets[n];
  nll[n] = (t >= 0 && t < vocab) ? (mm + __logf(ss)) - tgt[n] : 0.0f;
}

// H0[b, l, :] = emb[tokens[b, l], :]; ids outside [0, vocab) give a zero row.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ tokens,
                                                    const u32x4 *__restrict__ emb,
                                                    u32x4 *__restrict__ out, int vocab,
                                                    int cpr, int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / cpr;
  const int c = static_cast<int>(e - row * cpr);
  const int tok = tokens[row];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (tok >= 0 && tok < vocab) v = emb[static_cast<int64_t>(tok) * cpr + c];
  out[e] = v;
}

template <int E, int BM, int BN>
void launch_shape(const GemmParams &p, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>((p.rows + BM - 1) / BM) * (p.N / BN) *
                        (E == kEpiPartialF32 ? p.k_splits : 1);
  // slab width by measurement on the stack's shapes (K = 512..4096): with
  // loads two slabs ahead, 64-wide slabs win for every tile shape
  if (p.K % 64 == 0)
    hipLaunchKernelGGL((gemm_kernel<E, BM, BN, 64>), dim3(static_cast<unsigned>(tiles)), dim3(256),
                       0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<E, BM, BN, 32>), dim3(static_cast<unsigned>(tiles)), dim3(256),
                       0, s, p);
}

template <int E>
void launch_epi(const GemmParams &p, hipStream_t s) {
  if (E == kEpiLse) {  // the row tile must match lse_row_tiles
    if (p.N % 128 == 0)
      launch_shape<E, 128, 128>(p, s);
    else
      launch_shape<E, 128, 64>(p, s);
    return;
  }
  // by measurement on the stack's shapes: 128x128 tiles when they alone give
  // about two tiles per CU; split-K products 128x64 when the splits fill the
  // chip; the GELU product without the pre-activation store 128x128, else
  // 128x64, when they fill the chip (with the store, whose per-element
  // writes favour more, smaller tiles, 64x64); otherwise 64x64
  auto tiles = [&](int bm, int bn) {
    return static_cast<int64_t>((p.rows + bm - 1) / bm) * (p.N / bn) *
           (E == kEpiPartialF32 ? p.k_splits : 1);
  };
  const int64_t want = 512;
  const bool gelu_plain = E == kEpiGeluBf16 && !p.pre_out;
  if ((E != kEpiGeluBf16 || gelu_plain) && E != kEpiPartialF32 && p.N % 128 == 0 &&
      tiles(128, 128) >= want)
    launch_shape<E, 128, 128>(p, s);
  else if ((E == kEpiPartialF32 || gelu_plain) && tiles(128, 64) >= want)
    launch_shape<E, 128, 64>(p, s);
  else
    launch_shape<E, 64, 64>(p, s);
}

}  // namespace

txl_status launch_gemm(const GemmParams &p, int epi, hipStream_t s) {
  if (p.rows <= 0) return TXL_OK;
  if (p.K % 32 || p.N % 64 || (p.n_split < p.N && p.n_split % 128))
    return fail(TXL_ERR_UNSUPPORTED, "gemm: K must be a multiple of 32, N of 64 and the split of 128");
  if (p.c_seg < 0 || p.c_seg % 32)
    return fail(TXL_ERR_UNSUPPORTED, "gemm: output segment length must be a multiple of 32");
  if (epi == kEpiPartialF32 &&
      (p.k_splits < 1 || p.k_splits > p.K / 64 || p.n_split != p.N || p.gather))
    return fail(TXL_ERR_UNSUPPORTED, "gemm: split-K needs 1 <= splits <= K/64, no N split, no gather");
  const int64_t tiles = static_cast<int64_t>((p.rows + 63) / 64) * (p.N / 64) *
                        (epi == kEpiPartialF32 ? p.k_splits : 1);
  if (tiles > 0x7fffffffLL) return fail(TXL_ERR_UNSUPPORTED, "gemm: too many tiles");
  (void)hipGetLastError();
  if (epi == kEpiStoreBf16)
    launch_epi<kEpiStoreBf16>(p, s);
  else if (epi == kEpiGeluBf16)
    launch_epi<kEpiGeluBf16>(p, s);
  else if (epi == kEpiResidualF32)
    launch_epi<kEpiResidualF32>(p, s);
  else if (epi == kEpiPartialF32)
    launch_epi<kEpiPartialF32>(p, s);
  else if (epi == kEpiGeluGradBf16)
    launch_epi<kEpiGeluGradBf16>(p, s);
  else
    launch_epi<kEpiLse>(p, s);
  return check_launch("gemm_kernel");
}

txl_status launch_layernorm(const float *x, int n_parts, int64_t part_stride, const void *res,
                            const void *gamma, const void *beta, void *y, int rows, int d,
                            float eps, hipStream_t s, float *x_out) {
  if (rows <= 0) return TXL_OK;
  (void)hipGetLastError();
  const dim3 grid((rows + 3) / 4);
  const __bf16 *r = static_cast<const __bf16 *>(res);
  const __bf16 *g = static_cast<const __bf16 *>(gamma);
  const __bf16 *b = static_cast<const __bf16 *>(beta);
  __bf16 *o = static_cast<__bf16 *>(y);
  if (n_parts != 1 && n_parts != 2 && n_parts != 4)
    return fail(TXL_ERR_UNSUPPORTED, "layernorm: %d partial sums (1, 2 or 4 are built)", n_parts);
  auto go = [&](auto np) {
    constexpr int NP = decltype(np)::value;
    switch (d / 256) {
      case 1: hipLaunchKernelGGL((layernorm_kernel<NP, 1>), grid, dim3(256), 0, s, x, part_stride, r, g, b, o, rows, d, eps, x_out); break;
      case 2: hipLaunchKernelGGL((layernorm_kernel<NP, 2>), grid, dim3(256), 0, s, x, part_stride, r, g, b, o, rows, d, eps, x_out); break;
      case 3: hipLaunchKernelGGL((layernorm_kernel<NP, 3>), grid, dim3(256), 0, s, x, part_stride, r, g, b, o, rows, d, eps, x_out); break;
      case 4: hipLaunchKernelGGL((layernorm_kernel<NP, 4>), grid, dim3(256), 0, s, x, part_stride, r, g, b, o, rows, d, eps, x_out); break;
      default: hipLaunchKernelGGL((layernorm_kernel<NP, 0>), grid, dim3(256), 0, s, x, part_stride, r, g, b, o, rows, d, eps, x_out); break;
    }
  };
  if (n_parts == 1)
    go(std::integral_constant<int, 1>{});
  else if (n_parts == 2)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, 4>{});
  return check_launch("layernorm_kernel");
}

int lse_row_tiles(int rows, int /*N*/) { return (rows + 127) / 128; }

txl_status launch_lse_finish(const float *part_m, const float *part_s, const float *tgt,
                             const int32_t *targets, int n_tiles, int N, int vocab, float *nll,
                             hipStream_t s) {
  if (N <= 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(lse_finish_kernel, dim3((N + kFinTok - 1) / kFinTok), dim3(256), 0, s, part_m, part_s, tgt,
                     targets, n_tiles, N, vocab, nll);
  return check_launch("lse_finish_kernel");
}

txl_status launch_embed(const int32_t *tokens, const void *emb, void *out, int rows, int d,
                        int vocab, hipStream_t s) {
  const int cpr = d * 2 / 16;
  const int64_t total = static_cast<int64_t>(rows) * cpr;
  if (total == 0) return TXL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(embed_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                     s, tokens, static_cast<const u32x4 *>(emb), static_cast<u32x4 *>(out), vocab,
                     cpr, total);
  return check_launch("embed_kernel");
}

}  // namespace txl
