// FIFO memory as a ring buffer: append, per-row reset, logical read-out.
//
// [P1] "Transformer-XL" notes, "Segment-Level Recurrence": each layer's memory
// becomes Tail_M([mem; H]) after the step. [P4] "Transformer-XL": a FIFO
// buffer in GPU memory whose oldest states are overwritten. The ring writes
// only the L' = min(L, M) new rows into the slots that held the oldest ones,
// so an update moves 2*B*L'*d*s bytes instead of shifting all M rows.
//
// The copies are HBM-bound: each thread moves one 16-byte chunk of the
// flattened (ring, row, chunk) space, consecutive threads on consecutive
// chunks (whole 1 KiB spans per wavefront); the most waves in flight gave the
// best rate for updates of a few MB, where dispatch and ramp-up are a large
// part of the time. Row indices are split with multiply-shift division by
// host-computed magic numbers, and both streams carry non-temporal hints:
// neither side is reread soon.
#include <hip/hip_runtime.h>

#include "txl_internal.h"

namespace txl {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunks = 1;  // 16-byte chunks per thread (more per thread measured slower)

struct RingMeta {
  int B, M, L, Lp;
  uint32_t cpr;         // 16-byte chunks per row
  uint32_t src_cpr;     // 16-byte chunks between consecutive segment rows (>= cpr)
  FastDiv div_cpr, div_lp, div_b;
  uint32_t total;       // chunks in the launch
};

__global__ __launch_bounds__(kThreads) void mem_update_kernel(RingBatch rb, RingMeta mt) {
  const uint32_t base = blockIdx.x * (kThreads * kChunks) + threadIdx.x;
  u32x4 v[kChunks];
  u32x4 *dst[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const uint32_t e = base + j * kThreads;
    dst[j] = nullptr;
    if (e >= mt.total) continue;
    const uint32_t row = fdiv(e, mt.div_cpr);  // (ring, b, k) flattened
    const uint32_t c = e - row * mt.cpr;
    const uint32_t rk = fdiv(row, mt.div_lp);
    const uint32_t k = row - rk * mt.Lp;
    const uint32_t ring = fdiv(rk, mt.div_b);
    const uint32_t b = rk - ring * mt.B;
    // source row L - L' + k of segment row b; destination slot (head + k) mod M
    const int64_t src_row = static_cast<int64_t>(b) * mt.L + (mt.L - mt.Lp + k);
    int64_t slot = rb.head[ring] + k;
    if (slot >= mt.M) slot -= mt.M;
    const int64_t dst_row = static_cast<int64_t>(b) * mt.M + slot;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(rb.h[ring]) + src_row * mt.src_cpr + c;
    dst[j] = reinterpret_cast<u32x4 *>(rb.data[ring]) + dst_row * mt.cpr + c;
    v[j] = __builtin_nontemporal_load(src);
    if (k == 0 && c == 0) {
      const int nv = rb.valid[ring][b] + mt.L;
      rb.valid[ring][b] = nv < mt.M ? nv : mt.M;
    }
  }
#pragma unroll
  for (int j = 0; j < kChunks; ++j)
    if (dst[j]) __builtin_nontemporal_store(v[j], dst[j]);
}

// The same update when a row is a whole number of wavefronts (WPR waves of
// 64 chunks): the row, and with it the ring, batch row and slot, is uniform
// across a wavefront, so it is decoded once in scalar registers and each lane
// only adds its chunk index.
template <int WPR>
__global__ __launch_bounds__(kThreads) void mem_update_rows_kernel(RingBatch rb, RingMeta mt,
                                                                   uint32_t n_rows) {
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t row = __builtin_amdgcn_readfirstlane(wave / WPR);  // (ring, b, k) flattened
  if (row >= n_rows) return;
  const uint32_t c = (wave % WPR) * 64 + lane;
  const uint32_t rk = fdiv(row, mt.div_lp);
  const uint32_t k = row - rk * mt.Lp;
  const uint32_t ring = fdiv(rk, mt.div_b);
  const uint32_t b = rk - ring * mt.B;
  const int64_t src_row = static_cast<int64_t>(b) * mt.L + (mt.L - mt.Lp + k);
  int64_t slot = rb.head[ring] + k;
  if (slot >= mt.M) slot -= mt.M;
  const int64_t dst_row = static_cast<int64_t>(b) * mt.M + slot;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(rb.h[ring]) + src_row * mt.src_cpr + c;
  u32x4 *dst = reinterpret_cast<u32x4 *>(rb.data[ring]) + dst_row * mt.cpr + c;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src), dst);
  if (k == 0 && c == 0) {
    const int nv = rb.valid[ring][b] + mt.L;
    rb.valid[ring][b] = nv < mt.M ? nv : mt.M;
  }
}

// The same update for a single ring with its pointers passed directly: the
// pointer tables of the batched launch are a 1 KiB kernel argument, which a
// lone ring of a few MB pays for measurably. Two 16-byte chunks per thread
// (a workgroup covers 512 consecutive chunks), both loads in flight before
// the stores: a probe of copy shapes at 4-128 MB found this the fastest for
// 8-16 MiB copies (8 MiB: 3.9 us against 4.1 us with one chunk per thread
// and 4.7 us for the runtime's own copy), four chunks per thread slower.
constexpr int kOneChunks = 2;
__global__ __launch_bounds__(kThreads) void mem_update_one_kernel(u32x4 *__restrict__ data,
                                                                  const u32x4 *__restrict__ h,
                                                                  int32_t *__restrict__ valid,
                                                                  int64_t head, RingMeta mt) {
  const uint32_t base = blockIdx.x * (kThreads * kOneChunks) + threadIdx.x;
  u32x4 v[kOneChunks];
  u32x4 *dst[kOneChunks];
#pragma unroll
  for (int j = 0; j < kOneChunks; ++j) {
    const uint32_t e = base + j * kThreads;
    dst[j] = nullptr;
    if (e >= mt.total) continue;
    const uint32_t row = fdiv(e, mt.div_cpr);  // (b, k) flattened
    const uint32_t c = e - row * mt.cpr;
    const uint32_t b = fdiv(row, mt.div_lp);
    const uint32_t k = row - b * mt.Lp;
    const int64_t src_row = static_cast<int64_t>(b) * mt.L + (mt.L - mt.Lp + k);
    int64_t slot = head + k;
    if (slot >= mt.M) slot -= mt.M;
    const int64_t dst_row = static_cast<int64_t>(b) * mt.M + slot;
    v[j] = __builtin_nontemporal_load(h + src_row * mt.src_cpr + c);
    dst[j] = data + dst_row * mt.cpr + c;
    if (k == 0 && c == 0) {
      const int nv = valid[b] + mt.L;
      valid[b] = nv < mt.M ? nv : mt.M;
    }
  }
#pragma unroll
  for (int j = 0; j < kOneChunks; ++j)
    if (dst[j]) __builtin_nontemporal_store(v[j], dst[j]);
}

struct ValidPtrs {
  int32_t *p[kMaxRingsPerLaunch];
};

__global__ void mem_reset_kernel(ValidPtrs vp, int n, int B,
                                 const uint8_t *reset) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n * B) return;
  const int ring = e / B, b = e - ring * B;
  if (reset == nullptr || reset[b] != 0) vp.p[ring][b] = 0;
}

// valid[b] <- min(M, valid[b] + L) for every row of n caches (the count part
// of the ring update, for memories that hold projected keys and values)
__global__ void valid_advance_kernel(ValidPtrs vp, int n, int B, int M, int L) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n * B) return;
  const int ring = e / B, b = e - ring * B;
  const int nv = vp.p[ring][b] + L;
  vp.p[ring][b] = nv < M ? nv : M;
}

// Window compaction of projected-key/value caches: rows [start, start + M)
// of every batch row move to rows [0, M) (the caller guarantees start >= M,
// so source and destination never overlap). One 16-byte chunk per thread over
// the flattened (buffer, b, row, chunk) space.
struct KVCompactMeta {
  int M;
  int64_t cap, start;
  uint32_t cpr;
  FastDiv div_cpr, div_m, div_b;
  int B;
  uint32_t total;
};
__global__ __launch_bounds__(kThreads) void kv_compact_kernel(KVBuffers kb, KVCompactMeta mt) {
  const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= mt.total) return;
  const uint32_t row = fdiv(e, mt.div_cpr);  // (buffer, b, k) flattened
  const uint32_t c = e - row * mt.cpr;
  const uint32_t bk = fdiv(row, mt.div_m);
  const uint32_t k = row - bk * mt.M;
  const uint32_t buf = fdiv(bk, mt.div_b);
  const uint32_t b = bk - buf * mt.B;
  u32x4 *base = reinterpret_cast<u32x4 *>(kb.p[buf]);
  const int64_t brow = static_cast<int64_t>(b) * mt.cap;
  const u32x4 v = __builtin_nontemporal_load(base + (brow + mt.start + k) * mt.cpr + c);
  __builtin_nontemporal_store(v, base + (brow + k) * mt.cpr + c);
}

__global__ __launch_bounds__(kThreads) void mem_read_logical_kernel(
    const u32x4 *data, u32x4 *out, int M, int64_t head, uint32_t cpr, FastDiv div_cpr,
    FastDiv div_m, uint32_t total, const int32_t *valid_src, int32_t *valid_dst, int B) {
  if (valid_src && blockIdx.x == 0)  // the valid counts too, by the first workgroup
    for (int i = threadIdx.x; i < B; i += kThreads) valid_dst[i] = valid_src[i];
  const uint32_t base = blockIdx.x * (kThreads * kChunks) + threadIdx.x;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const uint32_t e = base + j * kThreads;
    if (e >= total) return;
    const uint32_t row = fdiv(e, div_cpr);  // (b, j') flattened
    const uint32_t c = e - row * cpr;
    const uint32_t b = fdiv(row, div_m);
    const uint32_t jl = row - b * M;
    int64_t slot = head + jl;
    if (slot >= M) slot -= M;
    out[static_cast<int64_t>(row) * cpr + c] = data[(static_cast<int64_t>(b) * M + slot) * cpr + c];
  }
}

}  // namespace

txl_status launch_mem_update(const RingBatch &rb, int n, int B, int M, int L,
                             int64_t row_bytes, int64_t src_row_bytes, hipStream_t s) {
  RingMeta mt;
  mt.B = B;
  mt.M = M;
  mt.L = L;
  mt.Lp = L < M ? L : M;
  const int64_t cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n) * B * mt.Lp * cpr;
  if (total >= (int64_t(1) << 31)) return fail(TXL_ERR_UNSUPPORTED, "mem_update: more than 2^31 chunks");
  mt.cpr = static_cast<uint32_t>(cpr);
  mt.src_cpr = static_cast<uint32_t>(src_row_bytes / 16);
  mt.div_cpr = make_fastdiv(mt.cpr);
  mt.div_lp = make_fastdiv(static_cast<uint32_t>(mt.Lp));
  mt.div_b = make_fastdiv(static_cast<uint32_t>(B));
  mt.total = static_cast<uint32_t>(total);
  const int64_t per_block = kThreads * kChunks;
  const unsigned blocks = static_cast<unsigned>((total + per_block - 1) / per_block);
  const uint32_t n_rows = static_cast<uint32_t>(total / cpr);
  (void)hipGetLastError();
  if (n == 1)
    hipLaunchKernelGGL(mem_update_one_kernel,
                       dim3(static_cast<unsigned>((total + kThreads * kOneChunks - 1) /
                                                  (kThreads * kOneChunks))),
                       dim3(kThreads), 0, s,
                       static_cast<u32x4 *>(rb.data[0]), static_cast<const u32x4 *>(rb.h[0]),
                       rb.valid[0], rb.head[0], mt);
  else if (cpr == 64)
    hipLaunchKernelGGL(mem_update_rows_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, rb, mt, n_rows);
  else if (cpr == 128)
    hipLaunchKernelGGL(mem_update_rows_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, rb, mt, n_rows);
  else
    hipLaunchKernelGGL(mem_update_kernel, dim3(blocks), dim3(kThreads), 0, s, rb, mt);
  return check_launch("mem_update_kernel");
}

txl_status launch_mem_reset(int32_t *const *valid, int n, int B,
                            const uint8_t *reset, hipStream_t s) {
  ValidPtrs vp;
  for (int i = 0; i < n; ++i) vp.p[i] = valid[i];
  const int total = n * B;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mem_reset_kernel, dim3((total + 255) / 256), dim3(256), 0, s, vp, n, B,
                     reset);
  return check_launch("mem_reset_kernel");
}

txl_status launch_valid_advance(int32_t *const *valid, int n, int B, int M, int L,
                                hipStream_t s) {
  ValidPtrs vp;
  for (int i = 0; i < n; ++i) vp.p[i] = valid[i];
  const int total = n * B;
  (void)hipGetLastError();
  hipLaunchKernelGGL(valid_advance_kernel, dim3((total + 255) / 256), dim3(256), 0, s, vp, n, B,
                     M, L);
  return check_launch("valid_advance_kernel");
}

txl_status launch_kv_compact(const KVBuffers &kb, int n, int B, int M, int64_t cap,
                             int64_t start, int64_t row_bytes, hipStream_t s) {
  KVCompactMeta mt;
  mt.M = M;
  mt.cap = cap;
  mt.start = start;
  mt.B = B;
  const int64_t cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n) * B * M * cpr;
  if (total == 0) return TXL_OK;
  if (total >= (int64_t(1) << 31)) return fail(TXL_ERR_UNSUPPORTED, "kv_compact: more than 2^31 chunks");
  mt.cpr = static_cast<uint32_t>(cpr);
  mt.div_cpr = make_fastdiv(mt.cpr);
  mt.div_m = make_fastdiv(static_cast<uint32_t>(M));
  mt.div_b = make_fastdiv(static_cast<uint32_t>(B));
  mt.total = static_cast<uint32_t>(total);
  (void)hipGetLastError();
  hipLaunchKernelGGL(kv_compact_kernel, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, kb, mt);
  return check_launch("kv_compact_kernel");
}

txl_status launch_mem_read_logical(const void *data, void *out, int B, int M,
                                   int64_t head, int64_t row_bytes,
                                   hipStream_t s, const int32_t *valid_src, int32_t *valid_dst) {
  const int64_t cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(B) * M * cpr;
  if (total >= (int64_t(1) << 31)) return fail(TXL_ERR_UNSUPPORTED, "mem_read_logical: more than 2^31 chunks");
  const int64_t per_block = kThreads * kChunks;
  const unsigned blocks = static_cast<unsigned>((total + per_block - 1) / per_block);
  (void)hipGetLastError();
  hipLaunchKernelGGL(mem_read_logical_kernel, dim3(blocks), dim3(kThreads), 0, s,
                     reinterpret_cast<const u32x4 *>(data), reinterpret_cast<u32x4 *>(out), M,
                     head, static_cast<uint32_t>(cpr), make_fastdiv(static_cast<uint32_t>(cpr)),
                     make_fastdiv(static_cast<uint32_t>(M)), static_cast<uint32_t>(total), valid_src,
                     valid_dst, B);
  return check_launch("mem_read_logical_kernel");
}

}  // namespace txl
