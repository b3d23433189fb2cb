// Relative-position attention, bf16 MFMA kernel for gfx950 (CDNA4).
//
// For query i and visible key position j ([P1] "Transformer-XL" notes,
// "Causal Mask With Memory": memory -valid <= j < 0, current 0 <= j <= i):
//   A_ij = (q_i + u).k_j + (q_i + v).R_{i-j}          ([P1] "Relative Positional
//          Encoding", regrouped as in [P3] section 2.2)
//   out_i = sum_j softmax_j(A_ij * scale) v_j         ([P1] "Dimension Walkthrough")
// R_{i-j} is row t = j' + L - 1 - i of the per-head table (j' = j + M).
//
// Design (one workgroup = 4 waves x 32 queries, key tiles of 64):
//  * Scores are computed transposed, S^T = K (Q')^T with the 32x32x16 bf16
//    MFMA, Q' = (q+u)*scale*log2(e) held in registers as the B operand. The
//    accumulator layout of S^T (one query per lane column, keys down the
//    registers) is exactly the B-operand layout that O^T = V^T P^T needs, so
//    the probabilities never leave registers.
//  * The position term uses the same trick with Q'' = (q+v)*scale*log2(e):
//    the band P[u][query] = R[t(u)] (Q'')^T covers the 95 distances one key
//    tile of one wave can need, as three 32-row MFMA blocks. The window
//    slides by 64 rows per key tile, so the last block of a tile is the first
//    block of the next: it is kept in registers, and each tile multiplies two
//    new blocks (two 32-row R loads, 8 MFMAs).
//  * The per-query diagonal read of the band (the relative shift, [P1]
//    "Relative Shift Trick" replaced by index arithmetic) goes through a
//    per-wave LDS band stored [u][query] with a row stride of 32 floats and
//    all 96 rows of the tile's three blocks (written once per tile, read by
//    both 32-key halves): lane r reads row c + 31 - r (+32 for the second
//    half) for key c, so both the write and the read put lane r on bank r.
//  * K and V tiles go from HBM straight into LDS with buffer-to-LDS loads
//    (16 bytes a lane, no registers), into two buffers: the next tile's
//    loads are issued at the top of a tile and waited for, with one barrier,
//    at its end. Rows are stored with their 16-byte chunks XOR-swizzled by
//    the row, which makes the K operand reads (16 bytes of one key row per
//    lane) and the transposing V reads (ds_read_b64_tr_b16, eight keys of
//    one dimension per lane for the V^T operand) free of LDS bank conflicts
//    (64 banks: 16 lanes of a 16-byte read, or 32 of an 8-byte read, must
//    cover all of them). R rows go straight from L2 into the A operand, one
//    tile ahead.
//  * The content MFMAs run first (their operands are in LDS when the tile
//    starts), while the band's results drain and its LDS round trip
//    completes; the shifted position term is then added to the scores.
//  * Masking: band row u of a tile is one distance for every query of the
//    wave, and the rows of negative distance (key after query) are exactly
//    the rows past a wave-uniform limit; on tiles that cross the diagonal
//    those rows are overwritten with -inf in LDS before the diagonal read,
//    so masked scores are -inf with no per-element compare.
//  * Online softmax in base 2 (scale folded into Q' and Q''). The running
//    max m is kept as long as every p = 2^(s - m) of a tile stays <= 2^8,
//    which is checked once per tile through each lane's sum of p (the sum
//    exceeds 2^8 whenever one p does); only then, and on the first tile, is
//    the row max taken (lane registers plus one exchange with lane^32) and
//    O, l rescaled. The row sum adds the fp32 p (the log-sum-exp handed to
//    the gradients keeps fp32 accuracy); PV uses p rounded to bf16.
//  * Key tiles run from the row's first valid memory slot to the
//    workgroup's diagonal. Query tiles are dealt heavier half first
//    (heaviest first), then the lighter half lightest first, so that a CU's
//    two resident workgroups pair a heavy tile with a light one; the
//    (batch, head) index varies fastest, so the tiles of one head land on
//    the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "txl_internal.h"

namespace txl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int DH = 64;         // head dimension served
constexpr int QW = 32;         // queries per wave (MFMA N)
constexpr int NW = 4;          // waves per workgroup
constexpr int BQ = QW * NW;    // queries per workgroup
constexpr int BK = 64;         // keys per tile
constexpr int NU = 3 * QW;     // band rows of a tile: key c of half kb reads u = c + 31 - r + 32kb < 95
constexpr int US = QW;         // band row stride (floats): the diagonal read puts lane r on bank r
constexpr float kPsumLimit = 256.0f;  // a tile keeps the running max while each lane's sum of p stays <= 2^8

// LDS: two K/V tile buffers (K [64 keys][64 dims] then V [64 keys][64 dims],
// bf16, 16-byte chunks swizzled: chunk c of key row n sits in slot c ^ kv_swz(n))
// and the waves' bands; 81920 bytes, two workgroups per CU.
constexpr int kTileElems = BK * DH;            // one K or V tile
constexpr int kBandFloats = NW * NU * US;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline bf16x8 load8(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ inline bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<__bf16>(0.0f);
  return z;
}

// Raw buffer loads: the hardware range check returns zeros for rows past the
// end of a buffer (and for negative offsets), so tile loads need no branches
// and the compiler can count outstanding loads exactly.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ inline u32x4 bload(rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}
// Non-temporal 16-byte copy through buffer loads / stores: an offset past the
// buffer's range loads zeros and stores nothing.
constexpr int kNonTemporal = 2;
constexpr int kOutOfRange = 0x7ffffff0;
constexpr int kAppendBatch = 8;  // ring-append chunks in flight per thread

// Counts a workgroup in a counter shared by n workgroups and returns the count
// before it; the count wraps to zero after the n-th, so the counter is zero
// again between launches. (The wrapping increment also keeps the compiler from
// turning the one-lane atomic into a wave reduction followed by a wait for
// every outstanding load.) Batch rows count apart, 256 bytes from each other:
// one counter for the whole grid cost 0.3 us more at B8 H16 L512 M512.
constexpr int kCounterStride = 64;  // uint32 per batch row's counter
__device__ inline uint32_t count_done(uint32_t *done, int n) {
  return __builtin_amdgcn_atomic_inc32(done, static_cast<uint32_t>(n - 1), __ATOMIC_RELAXED, "agent");
}
__device__ inline u32x4 bload_nt(rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, kNonTemporal));
}
__device__ inline void bstore_nt(rsrc_t rs, int byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, byte_off, 0, kNonTemporal);
}

typedef __attribute__((address_space(3))) void lds_void;

// Slot of chunk c of key row n (a row is 128 bytes, 8 slots; two rows span
// the 64 banks): c ^ kv_swz(n). The K operand read has 16 lanes read chunk c
// of rows n0 .. n0+15 at once, so the 8 even and the 8 odd rows each need 8
// distinct slots (bit 3 of n enters); the V read has 32 lanes read chunks
// 4db .. 4db+3 of rows n0+k, k < 4, so rows k and k+2 (same bank half) need
// slots in different groups of four (bit 1 of n flips bit 2).
__device__ inline int kv_swz(int n) { return (n & 7) ^ ((n << 1) & 4) ^ ((n >> 3) & 1); }

// Tile [j0, j0 + 64) of K and of V into an LDS buffer with direct
// buffer-to-LDS loads (no registers): wave w's instruction t = 2w + rep fills
// key rows 8t .. 8t+7, lane l landing at byte 16 l of that 1 KiB (row
// n = 8t + l/8, slot l % 8), so the lane loads source chunk
// (l % 8) ^ kv_swz(n) of its row. Rows past the buffer's range load zeros.
__device__ inline void dma_kv(rsrc_t krs, rsrc_t vrs, int row_bytes, int j0, __bf16 *buf, int wave,
                              int lane) {
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int t = 2 * wave + rep;
    const int row = 8 * t + (lane >> 3);
    const int off = (j0 + row) * row_bytes + 16 * ((lane & 7) ^ kv_swz(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(buf + 512 * t), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(buf + kTileElems + 512 * t), 16, off,
                                             0, 0, 0);
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
// Transposing LDS read: within each 16-lane group, element k of lane j is the
// 16-bit value at (address of lane 4k + j/4) + j % 4.
__device__ inline v4i16 lds_read_tr(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
}

// The attention of one query tile; with kAppend the workgroups of the lighter
// half of the query tiles also move the ring append's chunks once their key
// tiles are done. Each CU holds a light and a heavy workgroup side by side,
// and the light one's copy runs while the heavy one is still computing.
// (Copying inside the tile loop, one chunk per thread and tile, was slower:
// the tile loads, latency-critical here, then share the memory system with
// the copy, and a wave's wait for loads issued after a store also waits for
// that store. Counting the heavy workgroups in at their start instead of
// their end put the contended atomic's return on their first tile's wait.)
template <bool kAppend>
__device__ __forceinline__ void rel_attn_tile(const AttnParams &p, int n_qt, const RingAppend &ra,
                                              __bf16 *__restrict__ kv0, __bf16 *__restrict__ kv1,
                                              float *__restrict__ sband) {

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;   // query within the wave (MFMA column)
  const int hh = lane >> 5;  // which half of the wave

  // Query tiles: the heavier half first, heaviest first, then the lighter
  // half lightest first; a tile's key splits together; (batch, head)
  // fastest. When every workgroup is resident at once (two per CU), the
  // second workgroup a CU receives is then a light tile beside a heavy one
  // (key tiles 16 + 10 and 14 + 12 at L = 4 query tiles, not 16 + 12 and
  // 14 + 10).
  const int BH = p.B * p.H;
  const int S = p.n_split > 1 ? p.n_split : 1;
  const int unit = static_cast<int>(blockIdx.x) / BH;
  const int pos = unit / S, half_qt = (n_qt + 1) / 2;
  int qt = pos < half_qt ? n_qt - 1 - pos : pos - half_qt;
  // With three query tiles the third position pairs with the first on a CU
  // and the second runs alone when every workgroup is resident at once:
  // dealing the middle tile first pairs it with the lightest and leaves the
  // heaviest alone (key tiles 10 + 8 and 12 instead of 12 + 8 and 10; at
  // B16 H8 L384 M384 31.7 -> 29.6 us).
  if (n_qt == 3 && pos < 2) qt = pos == 0 ? 1 : 2;
  const int split = unit - (unit / S) * S;
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int L = p.L, M = p.M;
  const int i0 = qt * BQ;
  const int iw = i0 + wave * QW;
  const int i = iw + r;

  int valid = p.valid ? p.valid[b] : M;
  valid = valid < 0 ? 0 : (valid > M ? M : valid);
  const int j_vis = M - valid;                      // first visible key (logical)
  const int i_last = (i0 + BQ < L ? i0 + BQ : L) - 1;
  const int j_end = M + i_last + 1;                 // keys [j_vis, j_end) are staged
  // this workgroup's key tiles: all of them, or its split's contiguous share
  const int n_all = (j_end - j_vis + BK - 1) / BK;
  const int kt_b = split * n_all / S, kt_e = (split + 1) * n_all / S;
  const int j_lo = j_vis + kt_b * BK;               // first key of this workgroup
  const int n_tiles = kt_e - kt_b;
  const int ML = M + L;

  const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16 *kp = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *vp = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + h * p.kv_sh;
  const __bf16 *rp = static_cast<const __bf16 *>(p.r) + h * p.r_sh;
  const __bf16 *up = static_cast<const __bf16 *>(p.u) + h * DH;
  const __bf16 *vbp = static_cast<const __bf16 *>(p.vb) + h * DH;

  // keys [0, j_end) and R rows [0, M+L) are in range; the rest read as zero
  const int kv_row_bytes = static_cast<int>(p.kv_sl) * 2;
  const int r_row_bytes = static_cast<int>(p.r_sl) * 2;
  const rsrc_t krs = make_rsrc(kp, static_cast<uint32_t>((j_end - 1) * kv_row_bytes + 2 * DH));
  const rsrc_t vrs = make_rsrc(vp, static_cast<uint32_t>((j_end - 1) * kv_row_bytes + 2 * DH));
  const rsrc_t rrs = make_rsrc(rp, static_cast<uint32_t>((ML - 1) * r_row_bytes + 2 * DH));

  dma_kv(krs, vrs, kv_row_bytes, j_lo, kv0, wave, lane);

  // Q' = (q+u) c and Q'' = (q+v) c as B operands: k-step s holds dims 16s+8hh..+7
  const float c2 = p.scale * 1.4426950408889634f;
  bf16x8 qa[4], qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int d0 = 16 * s + 8 * hh;
    const bf16x8 qv = i < L ? load8(qp + static_cast<int64_t>(i) * p.q_sl + d0) : zero8();
    const bf16x8 uv = load8(up + d0);
    const bf16x8 vv = load8(vbp + d0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = static_cast<float>(qv[e]);
      qa[s][e] = static_cast<__bf16>((x + static_cast<float>(uv[e])) * c2);
      qb[s][e] = static_cast<__bf16>((x + static_cast<float>(vv[e])) * c2);
    }
  }

  const bool wave_active = iw < L;
  f32x16 o_acc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) o_acc[db][x] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  // This wave's band [u][r] starts at sband[band0]: written at u*US + r, the
  // shifted read of key c is [(c + 31 - r)][r]. LDS accesses index the
  // kernel's LDS arrays directly (one offset from the array), which lets the
  // compiler tell them apart from the tile buffer the loads are filling and
  // not wait for those loads before reading the band or the other buffer.
  const int band0 = wave * (NU * US);
  const int band_w = band0 + 4 * hh * US + r;
  const int band_r = band0 + (31 - r + 4 * hh) * US + r;

  // Band row u of the tile starting at key j0 is R row t = j0 + u + L - 32 - iw.
  // rr holds band blocks 1 and 2 (u = 32 + r, 64 + r) of the next tile, loaded
  // one tile ahead into the registers the band MFMAs have just freed; rows
  // outside [0, M+L) read as zero.
  bf16x8 rr[2][4];
  auto load_r = [&](int j0) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int off = (j0 + 32 * (bb + 1) + r + L - 32 - iw) * r_row_bytes + 16 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) rr[bb][s] = __builtin_bit_cast(bf16x8, bload(rrs, off + 32 * s));
    }
  };
  // band block 0 of the first tile; every later tile inherits it from the
  // previous tile's block 2 (the same R rows against the same queries)
  f32x16 b_carry;
  {
    bf16x8 r0[4];
    const int off = (j_lo + r + L - 32 - iw) * r_row_bytes + 16 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) r0[s] = __builtin_bit_cast(bf16x8, bload(rrs, off + 32 * s));
#pragma unroll
    for (int x = 0; x < 16; ++x) b_carry[x] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) b_carry = mfma32(r0[s], qb[s], b_carry);
  }
  load_r(j_lo);

  // V operand reads (transposing): lane l = 16g + 4k + q supplies the
  // address of V[key][d0 + 4q], key = 4hh + k (+ the k-step's base), so that
  // lane j of its group receives V[keys][d0 + j]; d0 = 32db + 16(g & 1).
  // Slot offsets of the swizzle: key = 4hh + k at the k-step's first eight
  // keys (a base that is a multiple of 16), 8 + 4hh + k at its second eight.
  int v_off[2], v_offh[2];
  {
    const int x = 4 * hh + ((lane >> 2) & 3);
    const int q = lane & 3;
    const int cc = 2 * ((lane >> 4) & 1) + (q >> 1);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      v_off[db] = x * DH + 8 * ((4 * db + cc) ^ kv_swz(x)) + 4 * (q & 1);
      v_offh[db] = x * DH + 8 * ((4 * db + cc) ^ kv_swz(x + 8)) + 4 * (q & 1);
    }
  }
  // K operand reads: key row n = 32kb + r, chunk 2s + hh in slot (2s + hh) ^ kv_swz(r)
  const int k_row = r * DH;

  // tile 0 in buffer 0 before the loop; every tile's loads are waited for
  // (with the R rows of the next tile) at the end of the tile before
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto run_tile = [&](int kt, const __bf16 *sk, __bf16 *nxt) {
    const int j0 = j_lo + kt * BK;
    // tile kt+1 into the other buffer (freed by the last barrier); past the
    // last tile the loads read zeros into a buffer nobody reads
    dma_kv(krs, vrs, kv_row_bytes, j0 + BK, nxt, wave, lane);
    // Every wave takes part in every tile's loads and barrier; a wave skips
    // the arithmetic of a tile past its last query's diagonal (the tile is
    // fully masked for it and would leave (m, l, O) unchanged; so are all
    // later tiles, so the band carry and the R prefetch are not needed).

    if (j0 <= M + iw + QW - 1) {  // some key of the tile is visible to this wave
      // ---- position band P[u][query] = R[t(u)] (Q'')^T, three blocks of 32 rows ----
      f32x16 b_acc[3];
      b_acc[0] = b_carry;
#pragma unroll
      for (int bb = 1; bb < 3; ++bb) {
#pragma unroll
        for (int x = 0; x < 16; ++x) b_acc[bb][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) b_acc[bb] = mfma32(rr[bb - 1][s], qb[s], b_acc[bb]);
      }
      b_carry = b_acc[2];
      // next tile's R rows into the registers just consumed
      load_r(j0 + BK);

      // Band row u of the tile is distance M - j0 - u + 31 + iw, so the rows
      // past the diagonal (negative distance, key after query) are the rows
      // u > ul0, the same for every query of the wave.
      const int ul0 = M - j0 + 31 + iw;

      // ---- scores S^T[key][query]: the accumulator starts from the shifted
      // position term and the content MFMA K (Q')^T adds onto it ----
      // register 4a+c' of block bb holds band row u = 32bb + 8a + 4hh + c'; the
      // three blocks go to rows 0..95 once, and the 32-key half kb reads rows
      // u = c + 31 - r + 32kb. Rows past the diagonal become -inf (masked keys
      // get weight exactly 0).
      // content scores first (their operands are in LDS since the tile
      // began), so they run while the band's results drain and its LDS
      // round trip completes; the shifted position term is added after
      f32x16 s_acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int x = 0; x < 16; ++x) s_acc[kb][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = load8(&sk[kb * 32 * DH + k_row + 8 * ((2 * s + hh) ^ kv_swz(r))]);
          s_acc[kb] = mfma32(a, qa[s], s_acc[kb]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < 3; ++bb)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            sband[band_w + (32 * bb + 8 * a4 + cc) * US] = b_acc[bb][4 * a4 + cc];
      if (ul0 < NU - 1) {
        const int start = (ul0 + 1 > 0 ? ul0 + 1 : 0) * US;
        const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        for (int f = start + 4 * lane; f < NU * US; f += 256)
          *reinterpret_cast<f32x4 *>(&sband[band0 + f]) = ninf;
      }
      wave_lds_sync();
      // all 16 two-dword diagonal reads are issued before the first add (left
      // to itself the compiler issued them two or three at a time, each
      // batch waiting for the LDS round trip of the one before)
      float dg[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int c = 8 * (x >> 2) + (x & 3);
          dg[kb][x] = sband[band_r + (c + 32 * kb) * US];
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // then the VALU adds
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) s_acc[kb][x] += dg[kb][x];

      // ---- online softmax in base 2 ----
      // p = 2^(s - m) with the running max m kept while every p of the tile
      // stays at most 2^8 (checked through the lane's sum of p, which exceeds
      // 2^8 whenever one p does); otherwise, and on the first tile, m moves to
      // the row's maximum so far and O, l are rescaled.
      bf16x8 pb[2][2];
      float psum;
      auto exp_tile = [&]() {
        psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pv = __builtin_amdgcn_exp2f(s_acc[kb][8 * s2 + e] - m_run);
              psum += pv;
              pb[kb][s2][e] = static_cast<__bf16>(pv);
            }
      };
      bool rescale = kt == 0;
      if (!rescale) {
        exp_tile();
        rescale = __builtin_amdgcn_ballot_w64(psum > kPsumLimit) != 0;
      }
      if (rescale) {
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) mt = fmaxf(mt, s_acc[kb][x]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        if (mt > m_run) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
          m_run = mt;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) o_acc[db][x] *= alpha;
        }
        exp_tile();
      }
      l_run += psum;

      // ---- O^T[d][query] += V^T P^T: k-step (kb, s2) covers keys kb*32 + 16 s2 + {4hh..4hh+3, 8+4hh..8+4hh+3} ----
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int vk = kTileElems + (kb * 32 + 16 * s2) * DH;
            const v4i16 lo = lds_read_tr(&sk[vk + v_off[db]]);
            const v4i16 hi = lds_read_tr(&sk[vk + 8 * DH + v_offh[db]]);
            // whole-vector cast: a per-element bit cast of these vectors was
            // folded to element 0 by the compiler
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o_acc[db] = mfma32(a, pb[kb][s2], o_acc[db]);
          }
    }
    // tile kt+1 (and the next R rows) landed; once every wave is here, it is
    // visible to all and tile kt's buffer is free for tile kt+2
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int kt = 0; kt < n_tiles; kt += 2) {
    run_tile(kt, kv0, kv1);
    if (kt + 1 < n_tiles) run_tile(kt + 1, kv1, kv0);
  }

  if constexpr (kAppend) {
    // Copy workers: the workgroups at dealing positions [copy_pos0,
    // copy_pos0 + copy_npos), the lighter query tiles. Worker thread g moves
    // chunks e = g + n * (worker threads), kAppendBatch rounds in flight at a
    // time; chunk e is byte 16c of new row k of batch row b
    // (e = (b L' + k) cpr + c), read from h row b L + L - L' + k and written
    // to ring slot (head + k) mod M.
    if (pos >= ra.copy_pos0 && pos < ra.copy_pos0 + ra.copy_npos) {
      const rsrc_t src_rs = make_rsrc(ra.h, ra.h_bytes);
      const rsrc_t dst_rs = make_rsrc(ra.data, ra.data_bytes);
      const uint32_t gid =
          static_cast<uint32_t>((pos - ra.copy_pos0) * BH + bh) * 256u + static_cast<uint32_t>(tid);
      const uint32_t step = ra.worker_threads;
      for (uint32_t n0 = 0; n0 < ra.rounds; n0 += kAppendBatch) {
        u32x4 val[kAppendBatch];
        int dst[kAppendBatch];
#pragma unroll
        for (int t = 0; t < kAppendBatch; ++t) {
          const uint32_t n = n0 + t;
          const uint32_t e = gid + n * step;
          const bool ok = n < ra.rounds && e < ra.total;
          const uint32_t ee = ok ? e : 0u;
          const uint32_t row = fdiv(ee, ra.div_cpr);
          const uint32_t c = ee - row * ra.cpr;
          const uint32_t bb = fdiv(row, ra.div_lp);
          const uint32_t k = row - bb * static_cast<uint32_t>(ra.Lp);
          const uint32_t src_row =
              bb * static_cast<uint32_t>(ra.L) + static_cast<uint32_t>(ra.L - ra.Lp) + k;
          uint32_t slot = static_cast<uint32_t>(ra.head) + k;
          if (slot >= static_cast<uint32_t>(ra.M)) slot -= static_cast<uint32_t>(ra.M);
          const uint32_t dst_row = bb * static_cast<uint32_t>(ra.M) + slot;
          val[t] = bload_nt(src_rs, ok ? static_cast<int>((src_row * ra.cpr + c) * 16u) : kOutOfRange);
          dst[t] = ok ? static_cast<int>((dst_row * ra.cpr + c) * 16u) : kOutOfRange;
        }
#pragma unroll
        for (int t = 0; t < kAppendBatch; ++t) bstore_nt(dst_rs, dst[t], val[t]);
      }
    }
    // Each workgroup counts itself in its batch row's counter at its end;
    // every thread of it read valid[b], and used it for its key range, before
    // the tile loop's barriers. The row's workgroup that counts last
    // therefore runs after every read of valid[b] in the grid: it advances
    // it. (The reads have returned before the increment is issued, so it
    // needs no release ordering, which would write back the L2.)
    if (tid == 0 && count_done(ra.done + kCounterStride * b, n_qt * p.H) == n_qt * p.H - 1) {
      const int nv = ra.valid[b] + ra.L;
      ra.valid[b] = nv < ra.M ? nv : ra.M;
    }
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (i >= L) return;
  if (S > 1) {  // partial result of this key range, merged by rel_attn_merge_kernel
    const int64_t row = (static_cast<int64_t>(split) * BH + bh) * L + i;
    float *po = p.part_o + row * DH;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 o4;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) o4[cc] = o_acc[db][4 * a4 + cc];
        *reinterpret_cast<f32x4 *>(po + db * 32 + 8 * a4 + 4 * hh) = o4;
      }
    if (hh == 0) {
      p.part_m[row] = m_run;
      p.part_l[row] = l_tot;
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  __bf16 *op = static_cast<__bf16 *>(p.out) + b * p.o_sb + h * p.o_sh + static_cast<int64_t>(i) * p.o_sl;
  // training also keeps the unrounded output
  float *o32 = p.out32 ? p.out32 + ((static_cast<int64_t>(b) * p.H + h) * L + i) * DH : nullptr;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      f32x4 of;
      bf16x4 o4;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        of[cc] = o_acc[db][4 * a4 + cc] * inv;
        o4[cc] = static_cast<__bf16>(of[cc]);
      }
      *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * a4 + 4 * hh) = o4;
      if (o32) *reinterpret_cast<f32x4 *>(o32 + db * 32 + 8 * a4 + 4 * hh) = of;
    }
  if (p.lse && hh == 0)
    p.lse[(static_cast<int64_t>(b) * p.H + h) * L + i] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
}

#define TXL_ATTN_LDS                                                  \
  __shared__ __attribute__((aligned(4096))) __bf16 kv0[2 * kTileElems]; \
  __shared__ __attribute__((aligned(4096))) __bf16 kv1[2 * kTileElems]; \
  __shared__ __attribute__((aligned(16))) float sband[kBandFloats];

__global__ __launch_bounds__(256, 2) void rel_attn_mfma_kernel(AttnParams p, int n_qt) {
  TXL_ATTN_LDS
  rel_attn_tile<false>(p, n_qt, RingAppend{}, kv0, kv1, sband);
}

__global__ __launch_bounds__(256, 2) void rel_attn_mfma_append_kernel(AttnParams p, int n_qt,
                                                                      RingAppend ra) {
  TXL_ATTN_LDS
  rel_attn_tile<true>(p, n_qt, ra, kv0, kv1, sband);
}
#undef TXL_ATTN_LDS

// Merge of the key-range splits: per query, m = max_s m_s and
// O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s (a split that saw no key
// has m_s = -inf and adds nothing). One thread per query and 4 dimensions.
// NS > 0: exactly NS splits, every split's m, l and O loaded before any is
// used (a loop over a run-time count waited for them one split at a time);
// NS = 0: any count. The sums run in split order either way.
template <int NS>
__global__ __launch_bounds__(256) void rel_attn_merge_kernel(AttnParams p) {
  const int64_t BHL = static_cast<int64_t>(p.B) * p.H * p.L;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= BHL * (DH / 4)) return;
  const int64_t row = e / (DH / 4);
  const int c = static_cast<int>(e - row * (DH / 4));
  float m = -INFINITY;
  float l = 0.0f;
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (NS > 0) {
    float ms[NS], ls[NS];
    f32x4 os[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      ms[sp] = p.part_m[sp * BHL + row];
      ls[sp] = p.part_l[sp * BHL + row];
      os[sp] = *reinterpret_cast<const f32x4 *>(p.part_o + (sp * BHL + row) * DH + 4 * c);
    }
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) m = fmaxf(m, ms[sp]);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      if (!(ms[sp] > -INFINITY)) continue;
      const float w = __builtin_amdgcn_exp2f(ms[sp] - m);
      l += w * ls[sp];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] += w * os[sp][q];
    }
  } else {
    for (int sp = 0; sp < p.n_split; ++sp) m = fmaxf(m, p.part_m[sp * BHL + row]);
    for (int sp = 0; sp < p.n_split; ++sp) {
      const float ms = p.part_m[sp * BHL + row];
      if (!(ms > -INFINITY)) continue;
      const float w = __builtin_amdgcn_exp2f(ms - m);
      l += w * p.part_l[sp * BHL + row];
      const f32x4 os = *reinterpret_cast<const f32x4 *>(p.part_o + (sp * BHL + row) * DH + 4 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] += w * os[q];
    }
  }
  const int64_t bh = row / p.L;
  const int i = static_cast<int>(row - bh * p.L);
  const int b = static_cast<int>(bh / p.H), h = static_cast<int>(bh - static_cast<int64_t>(b) * p.H);
  const float inv = 1.0f / l;
  bf16x4 o4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[q] *= inv;
    o4[q] = static_cast<__bf16>(o[q]);
  }
  __bf16 *op = static_cast<__bf16 *>(p.out) + b * p.o_sb + h * p.o_sh + static_cast<int64_t>(i) * p.o_sl;
  *reinterpret_cast<bf16x4 *>(op + 4 * c) = o4;
  if (p.out32) *reinterpret_cast<f32x4 *>(p.out32 + row * DH + 4 * c) = o;
  if (p.lse && c == 0) p.lse[row] = (m + log2f(l)) * 0.6931471805599453f;
}

// Zeroes the counters of n batch rows (kCounterStride apart).
__global__ __launch_bounds__(256) void counters_clear_kernel(uint32_t *done, int n) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < n) done[b * kCounterStride] = 0u;
}

}  // namespace

// The per-row counters of txl_rel_attn_fwd_mem_update_noalloc, for callers
// that cannot allocate: a file-scope device array, one copy per GPU, held
// until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) uint32_t scratch[kNoAllocMaxRows * kCounterStride];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

txl_status noalloc_counters(int B, hipStream_t s, uint32_t **out) {
  if (B > kNoAllocMaxRows)
    return fail(TXL_ERR_UNSUPPORTED,
                "rel_attn_mem_update_noalloc: B = %d exceeds the %d batch rows of the static counters",
                B, kNoAllocMaxRows);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(TXL_ERR_HIP, "rel_attn_mem_update_noalloc: no usable current device (%d)", dev);
  uint32_t *ptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void *p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(TXL_ERR_HIP, "rel_attn_mem_update_noalloc: hipGetSymbolAddress: %s",
                    hipGetErrorString(e));
      g_scratch_ptr[dev] = static_cast<uint32_t *>(p);
    }
    ptr = g_scratch_ptr[dev];
  }
  // every call starts from zeroed counters (a kernel, not a memset, so the
  // call can be captured in a graph); the attention launch leaves them zero
  (void)hipGetLastError();
  hipLaunchKernelGGL(counters_clear_kernel, dim3((B + 255) / 256), dim3(256), 0, s, ptr, B);
  const txl_status st = check_launch("counters_clear_kernel");
  if (st != TXL_OK) return st;
  *out = ptr;
  return TXL_OK;
}

// The kernels' LDS is static (81920 bytes, within the 160 KB of a CU for two
// workgroups); nothing to set up.
txl_status rel_attn_mfma_setup() { return TXL_OK; }

// Checks the shapes the buffer loads rely on and returns the grid (query
// tiles x splits x batch rows x heads).
static txl_status prepare_launch(const AttnParams &p, int *n_qt, int64_t *blocks) {
  // buffer loads address rows by 32-bit byte offsets from the (batch, head)
  // base and rely on rows not overlapping for the out-of-range zero fill
  if (p.kv_sl < DH || p.r_sl < DH || p.q_sl < DH || p.o_sl < DH)
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn: bf16 row strides must be >= d_h");
  const int64_t ML = static_cast<int64_t>(p.M) + p.L;
  // (the last tile's look-ahead loads reach up to two tiles past the keys)
  if ((ML + 2 * BK) * p.kv_sl * 2 >= (int64_t(1) << 31) || (ML + BK + QW) * p.r_sl * 2 >= (int64_t(1) << 31))
    return fail(TXL_ERR_UNSUPPORTED, "rel_attn: key / R rows span more than 2 GiB per head");
  *n_qt = (p.L + BQ - 1) / BQ;
  const int S = p.n_split > 1 ? p.n_split : 1;
  *blocks = static_cast<int64_t>(*n_qt) * p.B * p.H * S;
  if (*blocks > 0x7fffffffLL) return fail(TXL_ERR_UNSUPPORTED, "rel_attn: grid too large");
  return TXL_OK;
}

txl_status launch_rel_attn_mfma_append(const AttnParams &p, const RingAppend &ra, hipStream_t s) {
  if (p.n_split > 1) return fail(TXL_ERR_UNSUPPORTED, "rel_attn_append: key splits are not served");
  int n_qt;
  int64_t blocks;
  txl_status st = prepare_launch(p, &n_qt, &blocks);
  if (st != TXL_OK) return st;
  // Copy workers: the lighter half of the query tiles (dealt after the
  // heavier half), or every tile when there is one. (Measured at B8 H16
  // L512 M512: the lightest quarter alone, or every workgroup, copied
  // slower; so did 2, 4 or 16 chunks in flight per thread instead of 8.)
  // Chunk indices g + n * threads stay below 2^32 while the grid's thread
  // count and the chunk count are both below 2^31.
  const int64_t threads = blocks * 256;
  const int copy_pos0 = n_qt > 1 ? (n_qt + 1) / 2 : 0;
  const int copy_npos = n_qt > 1 ? n_qt - copy_pos0 : 1;
  const int64_t workers = static_cast<int64_t>(copy_npos) * p.B * p.H * 256;
  if (threads >= (int64_t(1) << 31)) {  // the two as separate launches
    st = launch_rel_attn_mfma(p, s);
    if (st != TXL_OK) return st;
    RingBatch rb;
    rb.data[0] = ra.data;
    rb.valid[0] = ra.valid;
    rb.h[0] = ra.h;
    rb.head[0] = ra.head;
    return launch_mem_update(rb, 1, ra.B, ra.M, ra.L, static_cast<int64_t>(ra.cpr) * 16,
                             static_cast<int64_t>(ra.cpr) * 16, s);
  }
  RingAppend a = ra;
  a.copy_pos0 = copy_pos0;
  a.copy_npos = copy_npos;
  a.worker_threads = static_cast<uint32_t>(workers);
  a.rounds = static_cast<uint32_t>((static_cast<int64_t>(a.total) + workers - 1) / workers);
  (void)hipGetLastError();
  hipLaunchKernelGGL(rel_attn_mfma_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, s, p, n_qt, a);
  return check_launch("rel_attn_mfma_append_kernel");
}

txl_status launch_rel_attn_mfma(const AttnParams &p, hipStream_t s) {
  int n_qt;
  int64_t blocks;
  txl_status st0 = prepare_launch(p, &n_qt, &blocks);
  if (st0 != TXL_OK) return st0;
  const int S = p.n_split > 1 ? p.n_split : 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(rel_attn_mfma_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, s, p, n_qt);
  txl_status st = check_launch("rel_attn_mfma_kernel");
  if (st != TXL_OK || S == 1) return st;
  const int64_t threads = static_cast<int64_t>(p.B) * p.H * p.L * (DH / 4);
  const dim3 mgrid(static_cast<unsigned>((threads + 255) / 256));
  if (S == 2)
    hipLaunchKernelGGL(rel_attn_merge_kernel<2>, mgrid, dim3(256), 0, s, p);
  else if (S == 3)
    hipLaunchKernelGGL(rel_attn_merge_kernel<3>, mgrid, dim3(256), 0, s, p);
  else if (S == 4)
    hipLaunchKernelGGL(rel_attn_merge_kernel<4>, mgrid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(rel_attn_merge_kernel<0>, mgrid, dim3(256), 0, s, p);
  return check_launch("rel_attn_merge_kernel");
}

}  // namespace txl
