// Weight-gradient products of the stack's backward: out = X^T Y, where X
// [K, rows] and Y [K, N] are activations or output gradients stored one
// segment row per row (the reduction runs over the segment's rows, the
// strided dimension of both operands).
//
// [P1] "Transformer-XL" notes, "Training Loop Sketch": a segment's loss is
// back-propagated through the segment alone, so every weight gradient of a
// layer is a sum over the segment's B*L rows (over the B*(M+L) key rows for
// W^K and W^V, whose memory part is a constant input, and over the M+L
// distances for W_R).
//
// Both operands stay in the layout the forward wrote: 64-row slabs of X
// and Y go straight from global memory into LDS with direct buffer-to-LDS
// loads (16 bytes a lane, [k][column] order, no registers), and the MFMA
// operands, which need eight consecutive k of one column per lane, come out
// of LDS with transposing reads (ds_read_b64_tr_b16). Workgroups of 4 waves
// compute 128 x 128 (or 64 x 64) output tiles with v_mfma_f32_32x32x16_bf16,
// two LDS buffers with one barrier per slab, and the K range split over
// k_splits workgroups whose fp32 partials are added afterwards in split
// order (a fixed order: the result does not depend on scheduling). The
// products of a layer run as one batch: a launch's workgroups are dealt to
// the products in turn, so the splits need only fill the chip together.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "txl_internal.h"

namespace txl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;
constexpr int KS = 64;  // k rows per slab

// One product of a launch: its workgroups are [wg_begin, wg_begin + tiles
// k_splits) of the grid, split s taking [wg_begin + s tiles, ...).
struct DwJob {
  const __bf16 *x, *y;
  float *out;
  int64_t ldx, ldy, split_stride;
  int rows, N, k_rows, k_splits, tiles, wg_begin;
};
struct DwBatch {
  DwJob job[kMaxDwProblems];
  int n;
};

// The split products' partial sums, all in one launch: product j owns the
// threads [e_begin, e_begin + n4) (e_begin a multiple of 256, so a
// workgroup serves one product), four floats a thread.
struct DwRed {
  const float *part;
  float *out;
  int64_t n4, e_begin;
  int S;
};
struct DwRedBatch {
  DwRed job[kMaxDwProblems];
  int n;
};

__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Transposing LDS read: within each 16-lane group, element e of lane j is
// the 16-bit value at (address of lane 4e + j/4) + j % 4.
__device__ inline v4i16 lds_read_tr(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
}

// Slab layout in LDS: row k (KS rows) of W columns, the row's 16-byte
// chunk c at slot c ^ swz(k). A transposing read of one MFMA operand
// touches rows k0 + {0..3} and k0 + {8..11} (k0 a multiple of 4), four
// chunks each; swz spreads the rows k0 + e over distinct banks, so every
// bank serves four 4-byte reads, the minimum for 512 bytes.
template <int W>
__device__ inline int swz(int k) {
  return (4 * (k & 3)) & (W / 8 - 1);
}

// One slab (rows [kb, kb + KS) of the operand, columns [c0, c0 + W)) into
// LDS: instruction t of wave w fills bytes [1024 t, 1024 t + 1024) of the
// slab, lane l landing at byte 16 l of them. Rows past the resource's range
// load zeros.
template <int W>
__device__ inline void dma_slab(rsrc_t rs, int row_bytes, __bf16 *dst, int wave, int lane) {
  constexpr int CPR = W / 8;          // chunks per row
  constexpr int RPI = 512 / W;        // rows per instruction
  constexpr int PER_WAVE = W / 32;    // instructions per wave (W / 8 in all)
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int t = wave * PER_WAVE + i;
    const int row = t * RPI + lane / CPR;
    const int slot = lane % CPR;
    const int off = row * row_bytes + 16 * (slot ^ swz<W>(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + 512 * t), 16, off, 0, 0, 0);
  }
}

// The slab rows [kb, kb + KS) of an operand whose rows [0, k_rows) exist:
// a resource starting at row kb, column c0, covering up to the last
// existing row's W columns (empty past the end).
template <int W>
__device__ inline rsrc_t slab_rsrc(const __bf16 *base, int64_t ld, int c0, int kb, int k_rows) {
  const int rem = k_rows - kb;
  const int n = rem < KS ? rem : KS;
  const uint32_t bytes = n > 0 ? static_cast<uint32_t>((n - 1) * ld * 2 + W * 2) : 0u;
  return make_rsrc(base + static_cast<int64_t>(kb) * ld + c0, bytes);
}

template <int BM, int BN>
__global__ __launch_bounds__(256, 2) void dw_kernel(DwBatch bt) {
  constexpr int WM = BM / 64, WN = BN / 64;  // 32 x 32 blocks per wave
  __shared__ __attribute__((aligned(4096))) __bf16 sx0[KS * BM];
  __shared__ __attribute__((aligned(4096))) __bf16 sx1[KS * BM];
  __shared__ __attribute__((aligned(4096))) __bf16 sy0[KS * BN];
  __shared__ __attribute__((aligned(4096))) __bf16 sy1[KS * BN];

  // XCD-contiguous workgroup order (a bijection on [0, T)), then the
  // product owning the index (a wave-uniform choice among the batch's
  // entries, made with constant indices so the entries stay scalar)
  const int T = gridDim.x;
  const int bid = blockIdx.x;
  const int xc = bid % kXcds, local = bid / kXcds;
  const int q = T / kXcds, rem = T % kXcds;
  const int gidx = xc * q + (xc < rem ? xc : rem) + local;
  DwJob J = bt.job[0];
#pragma unroll
  for (int k = 1; k < kMaxDwProblems; ++k)
    if (k < bt.n && gidx >= bt.job[k].wg_begin) J = bt.job[k];
  const __bf16 *__restrict__ x = J.x;
  const __bf16 *__restrict__ y = J.y;
  const int64_t ldx = J.ldx, ldy = J.ldy;
  const int N = J.N, k_rows = J.k_rows, k_splits = J.k_splits;
  int tile = gidx - J.wg_begin;
  const int split = tile / J.tiles;
  tile -= split * J.tiles;
  const int n_tn = N / BN;
  const int tm = tile / n_tn, tn = tile - tm * n_tn;
  const int m0 = tm * BM, n0 = tn * BN;

  const int n_slabs = (k_rows + KS - 1) / KS;
  const int ks0 = static_cast<int>(static_cast<int64_t>(split) * n_slabs / k_splits);
  const int ks1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_slabs / k_splits);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // transposing-read offsets (elements, k-step 0, first half): lane
  // 16g + 4e + qq supplies row 8 (g >> 1) + e, columns 16 (g & 1) + 4 qq of
  // a 32-column block; the second half reads rows + 4, k-step s rows + 16 s
  const int g = lane >> 4, e = (lane >> 2) & 3, qq = lane & 3;
  const int kr = 8 * (g >> 1) + e;
  int xo[WM], yo[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int m = wm * (BM / 2) + 32 * i + 16 * (g & 1) + 4 * qq;
    xo[i] = kr * BM + 8 * ((m >> 3) ^ swz<BM>(kr)) + (m & 7);
  }
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int n = wn * (BN / 2) + 32 * j + 16 * (g & 1) + 4 * qq;
    yo[j] = kr * BN + 8 * ((n >> 3) ^ swz<BN>(kr)) + (n & 7);
  }
  // rows kr + 4 h + 16 s all have (row & 3) == e: the swizzle is the same

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int xrb = static_cast<int>(ldx * 2), yrb = static_cast<int>(ldy * 2);
  auto load = [&](int ks, __bf16 *dx, __bf16 *dy) {
    dma_slab<BM>(slab_rsrc<BM>(x, ldx, m0, ks * KS, k_rows), xrb, dx, wave, lane);
    dma_slab<BN>(slab_rsrc<BN>(y, ldy, n0, ks * KS, k_rows), yrb, dy, wave, lane);
  };
  auto compute = [&](const __bf16 *cx, const __bf16 *cy) {
#pragma unroll
    for (int s = 0; s < KS / 16; ++s) {
      bf16x8 a[WM], b[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const v4i16 lo = lds_read_tr(cx + xo[i] + 16 * s * BM);
        const v4i16 hi = lds_read_tr(cx + xo[i] + (16 * s + 4) * BM);
        a[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const v4i16 lo = lds_read_tr(cy + yo[j] + 16 * s * BN);
        const v4i16 hi = lds_read_tr(cy + yo[j] + (16 * s + 4) * BN);
        b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Slab ks sits in buffer (ks - ks0) % 2. The wait and barrier at the top
  // of a slab make its loads visible and free the other buffer (read during
  // the slab before), which then takes slab ks + 1 while this one computes.
  if (ks0 < ks1) load(ks0, sx0, sy0);
  for (int ks = ks0; ks < ks1; ks += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ks + 1 < ks1) load(ks + 1, sx1, sy1);
    compute(sx0, sy0);
    if (ks + 1 >= ks1) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ks + 2 < ks1) load(ks + 2, sx0, sy0);
    compute(sx1, sy1);
  }

  // register 4 a + c of block (i, j) holds out[m0 + wm BM/2 + 32 i + 8 a +
  // 4 (lane / 32) + c][n0 + wn BN/2 + 32 j + lane % 32]
  float *o = J.out + split * J.split_stride;
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int col = n0 + wn * (BN / 2) + 32 * j + r;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int row = m0 + wm * (BM / 2) + 32 * i + 8 * a + 4 * hh + c;
          o[static_cast<int64_t>(row) * N + col] = acc[i][j][4 * a + c];
        }
    }
}

// out[i] = sum_{s < S} part[s * n + i] (n = 4 n4), s ascending. The parts
// are loaded eight at a time (the index clamped to the last part, so the
// loads need no branch) before any of them is added: one load at a time
// left a thread waiting a full memory round trip per part.
constexpr int kPartBatch = 8;
__global__ __launch_bounds__(256) void dw_reduce_kernel(DwRedBatch rb) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t gidx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  DwRed R = rb.job[0];
#pragma unroll
  for (int k = 1; k < kMaxDwProblems; ++k)
    if (k < rb.n && gidx >= rb.job[k].e_begin) R = rb.job[k];
  const int64_t e = gidx - R.e_begin;
  if (e >= R.n4) return;
  const f32x4 *p = reinterpret_cast<const f32x4 *>(R.part) + e;
  f32x4 acc = p[0];
  for (int s0 = 1; s0 < R.S; s0 += kPartBatch) {
    f32x4 v[kPartBatch];
#pragma unroll
    for (int t = 0; t < kPartBatch; ++t) v[t] = p[(s0 + t < R.S ? s0 + t : R.S - 1) * R.n4];
#pragma unroll
    for (int t = 0; t < kPartBatch; ++t)
      if (s0 + t < R.S) acc += v[t];
  }
  reinterpret_cast<f32x4 *>(R.out)[e] = acc;
}

}  // namespace

// 128 x 128 tiles when the output divides into them, else 64 x 64.
static bool dw_big_tiles(int rows, int N) { return rows % 128 == 0 && N % 128 == 0; }

// Splits of a batch: every split of every product should carry about the
// same work, total / kDwTargetWgs, where a product's work is its tiles x K
// slabs (a 64 x 64 tile counts a quarter of a 128 x 128 one); at least one
// slab per split, at most 64 splits.
constexpr int64_t kDwTargetWgs = 512;
static void dw_plan(const DwProblem *p, int n, int *splits) {
  int64_t total = 0;  // in quarter tile-slabs (a 64 x 64 tile and one slab)
  for (int j = 0; j < n; ++j) {
    const int tm = dw_big_tiles(p[j].rows, p[j].N) ? 128 : 64;
    const int64_t tiles = static_cast<int64_t>(p[j].rows / tm) * (p[j].N / tm);
    const int64_t slabs = (p[j].k_rows + KS - 1) / KS;
    total += tiles * slabs * (tm == 128 ? 4 : 1);
  }
  int64_t per = total / kDwTargetWgs;  // quarter tile-slabs per workgroup
  if (per < 1) per = 1;
  for (int j = 0; j < n; ++j) {
    const int q = dw_big_tiles(p[j].rows, p[j].N) ? 4 : 1;
    const int64_t slabs = (p[j].k_rows + KS - 1) / KS;
    int64_t sp = (slabs * q + per / 2) / per;
    if (sp > slabs) sp = slabs;
    if (sp > 64) sp = 64;
    splits[j] = sp < 1 ? 1 : static_cast<int>(sp);
  }
}

size_t dw_batch_part_floats(const DwProblem *p, int n) {
  if (n < 1 || n > kMaxDwProblems) return 0;
  int sp[kMaxDwProblems];
  dw_plan(p, n, sp);
  size_t f = 0;
  for (int j = 0; j < n; ++j)
    if (sp[j] > 1) f += static_cast<size_t>(sp[j]) * p[j].rows * p[j].N;
  return f;
}

txl_status launch_dw_batch(const DwProblem *p, int n, float *part, size_t part_floats,
                           hipStream_t s) {
  if (n < 1 || n > kMaxDwProblems) return fail(TXL_ERR_INVALID_ARG, "dw_batch: %d products", n);
  for (int j = 0; j < n; ++j) {
    const DwProblem &d = p[j];
    if (d.rows < 0 || d.N < 0 || d.k_rows < 0 || d.rows % 64 || d.N % 64)
      return fail(TXL_ERR_INVALID_ARG, "dw_gemm: rows %d and N %d must be multiples of 64, k_rows %d >= 0",
                  d.rows, d.N, d.k_rows);
    if (d.rows == 0 || d.N == 0) continue;
    if (!d.x || !d.y || !d.out || d.ldx < d.rows || d.ldy < d.N || d.ldx % 8 || d.ldy % 8 ||
        reinterpret_cast<uintptr_t>(d.x) % 16 || reinterpret_cast<uintptr_t>(d.y) % 16)
      return fail(TXL_ERR_INVALID_ARG, "dw_gemm: operands must be 16-byte aligned with ldx >= rows, "
                                   "ldy >= N, strides multiples of 8");
    // a slab's resource spans up to 64 rows: offsets within it fit 32 bits
    if (static_cast<int64_t>(KS) * (d.ldx > d.ldy ? d.ldx : d.ldy) * 2 >= (int64_t{1} << 31))
      return fail(TXL_ERR_UNSUPPORTED, "dw_gemm: row stride too large");
  }
  const size_t need = dw_batch_part_floats(p, n);
  if (need > 0 && (!part || part_floats < need))
    return fail(TXL_ERR_WORKSPACE, "dw_batch: %zu partial floats < %zu", part_floats, need);
  int sp[kMaxDwProblems];
  dw_plan(p, n, sp);
  // one launch per tile shape
  DwBatch big = {}, small = {};
  int64_t wg_big = 0, wg_small = 0;
  size_t poff = 0;
  for (int j = 0; j < n; ++j) {
    const DwProblem &d = p[j];
    if (d.rows == 0 || d.N == 0) continue;
    const bool b = dw_big_tiles(d.rows, d.N);
    const int tm = b ? 128 : 64;
    DwJob J;
    J.x = static_cast<const __bf16 *>(d.x);
    J.y = static_cast<const __bf16 *>(d.y);
    J.ldx = d.ldx;
    J.ldy = d.ldy;
    J.rows = d.rows;
    J.N = d.N;
    J.k_rows = d.k_rows;
    J.k_splits = sp[j];
    J.tiles = (d.rows / tm) * (d.N / tm);
    J.split_stride = static_cast<int64_t>(d.rows) * d.N;
    J.out = sp[j] > 1 ? part + poff : d.out;
    if (sp[j] > 1) poff += static_cast<size_t>(sp[j]) * d.rows * d.N;
    DwBatch &B = b ? big : small;
    int64_t &wg = b ? wg_big : wg_small;
    J.wg_begin = static_cast<int>(wg);
    wg += static_cast<int64_t>(J.tiles) * sp[j];
    B.job[B.n++] = J;
  }
  if (wg_big > 0x7fffffff || wg_small > 0x7fffffff) return fail(TXL_ERR_UNSUPPORTED, "dw_gemm: too many tiles");
  (void)hipGetLastError();
  if (big.n)
    hipLaunchKernelGGL((dw_kernel<128, 128>), dim3(static_cast<unsigned>(wg_big)), dim3(256), 0, s, big);
  if (small.n)
    hipLaunchKernelGGL((dw_kernel<64, 64>), dim3(static_cast<unsigned>(wg_small)), dim3(256), 0, s, small);
  txl_status st = check_launch("dw_kernel");
  if (st != TXL_OK) return st;
  // the split products' partials, each summed in split order, one launch
  DwRedBatch rb = {};
  int64_t threads = 0;
  poff = 0;
  for (int j = 0; j < n; ++j) {
    const DwProblem &d = p[j];
    if (d.rows == 0 || d.N == 0 || sp[j] == 1) continue;
    DwRed R;
    R.part = part + poff;
    R.out = d.out;
    R.n4 = static_cast<int64_t>(d.rows) * d.N / 4;
    R.S = sp[j];
    R.e_begin = threads;
    threads += (R.n4 + 255) / 256 * 256;
    rb.job[rb.n++] = R;
    poff += static_cast<size_t>(sp[j]) * d.rows * d.N;
  }
  if (rb.n == 0) return TXL_OK;
  if (reinterpret_cast<uintptr_t>(part) % 16)
    return fail(TXL_ERR_UNSUPPORTED, "dw_batch: partials must be 16-byte aligned");
  for (int j = 0; j < rb.n; ++j)
    if (reinterpret_cast<uintptr_t>(rb.job[j].out) % 16)
      return fail(TXL_ERR_UNSUPPORTED, "dw_batch: split product outputs must be 16-byte aligned");
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(static_cast<unsigned>(threads / 256)), dim3(256), 0, s, rb);
  return check_launch("dw_reduce_kernel");
}

}  // namespace txl
