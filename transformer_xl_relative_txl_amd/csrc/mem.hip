// FIFO memory as a ring buffer: append, per-row reset, logical read-out.
//
// [P1] "Transformer-XL" notes, "Segment-Level Recurrence": each layer's memory
// becomes Tail_M([mem; H]) after the step. [P4] "Transformer-XL": a FIFO
// buffer in GPU memory whose oldest states are overwritten. The ring writes
// only the L' = min(L, M) new rows into the slots that held the oldest ones,
// so an update moves 2*B*L'*d*s bytes instead of shifting all M rows.
//
// All three kernels are plain 16-byte copies: one uint4 per thread, rows
// contiguous in memory, consecutive threads on consecutive 16-byte chunks of
// a row, so every wavefront reads and writes whole 1 KiB spans.
#include <hip/hip_runtime.h>

#include "txl_internal.h"

namespace txl {
namespace {

struct RingMeta {
  int B, M, L, Lp;
  int64_t cpr;  // 16-byte chunks per row
};

__global__ __launch_bounds__(256) void mem_update_kernel(RingBatch rb,
                                                         RingMeta mt,
                                                         int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / mt.cpr;  // (ring, b, k) flattened
  const int64_t c = e - row * mt.cpr;
  const int k = static_cast<int>(row % mt.Lp);
  const int64_t rb_ = row / mt.Lp;
  const int b = static_cast<int>(rb_ % mt.B);
  const int ring = static_cast<int>(rb_ / mt.B);
  // source row L - L' + k of segment row b; destination slot (head + k) mod M
  const int64_t src_row = static_cast<int64_t>(b) * mt.L + (mt.L - mt.Lp + k);
  const int64_t slot = (rb.head[ring] + k) % mt.M;
  const int64_t dst_row = static_cast<int64_t>(b) * mt.M + slot;
  const uint4 *src = reinterpret_cast<const uint4 *>(rb.h[ring]) + src_row * mt.cpr + c;
  uint4 *dst = reinterpret_cast<uint4 *>(rb.data[ring]) + dst_row * mt.cpr + c;
  *dst = *src;
  if (k == 0 && c == 0) {
    const int v = rb.valid[ring][b] + mt.L;
    rb.valid[ring][b] = v < mt.M ? v : mt.M;
  }
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

__global__ __launch_bounds__(256) void mem_read_logical_kernel(
    const uint4 *data, uint4 *out, int M, int64_t head, int64_t cpr,
    int64_t total) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t row = e / cpr;  // (b, j') flattened
  const int64_t c = e - row * cpr;
  const int64_t b = row / M;
  const int64_t j = row - b * M;
  const int64_t slot = (head + j) % M;
  out[row * cpr + c] = data[(b * M + slot) * cpr + c];
}

}  // namespace

txl_status launch_mem_update(const RingBatch &rb, int n, int B, int M, int L,
                             int64_t row_bytes, hipStream_t s) {
  RingMeta mt;
  mt.B = B;
  mt.M = M;
  mt.L = L;
  mt.Lp = L < M ? L : M;
  mt.cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n) * B * mt.Lp * mt.cpr;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return fail(TXL_ERR_UNSUPPORTED, "mem_update: too many rows");
  (void)hipGetLastError();
  hipLaunchKernelGGL(mem_update_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     rb, mt, total);
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

txl_status launch_mem_read_logical(const void *data, void *out, int B, int M,
                                   int64_t head, int64_t row_bytes,
                                   hipStream_t s) {
  const int64_t cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(B) * M * cpr;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return fail(TXL_ERR_UNSUPPORTED, "mem_read_logical: too many rows");
  (void)hipGetLastError();
  hipLaunchKernelGGL(mem_read_logical_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     s, reinterpret_cast<const uint4 *>(data), reinterpret_cast<uint4 *>(out), M,
                     head, cpr, total);
  return check_launch("mem_read_logical_kernel");
}

}  // namespace txl
