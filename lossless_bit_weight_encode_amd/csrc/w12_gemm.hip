// W12 GEMM: Y[M][N] = X[M][K] . W[N][K]^T with BF16 X, W12 weights and FP32 accumulation.
//
// SpecPilot summary page, method bullet of section 4.1: the W12 GEMM is a stream-K GEMM that
// decodes the records in registers and splits the reduction in a fixed order, so it is
// deterministic.  This gfx950 version:
//   * streams the hi/lo record planes from HBM into a per-wave two-stage LDS ring with
//     buffer-to-LDS DMA loads (no registers held while a stage is in flight), reads each
//     lane's 16 + 8 bytes back, decodes them to BF16 pairs in registers (decode16) and
//     patches the escapes of the lane's own k range through a cursor over its channel's
//     ascending escape list;
//   * M <= 8: FP32 dot2 (v_dot2c_f32_bf16) accumulation per lane, a fixed butterfly over the
//     4 lane groups and a fixed wave order through LDS (wavefront GEMV); X rides the ring;
//   * M >= 9: the decoded chunk is the B operand of v_mfma_f32_16x16x32_bf16 (16 rows of W x
//     32 k) and X rows (padded to 16) are the A operand, double-buffered in registers;
//   * schedules work stream-K style: the grid is the number of work-groups resident at once,
//     and work-group w takes the contiguous range [w U / G, (w+1) U / G) of the U = tiles x
//     units work units (a unit is 16 chunks of one tile), so every work-group streams the
//     same number of bytes.  A tile covered by several work-groups gets one partial per
//     segment; the last segment to finish sums them in segment order (a fixed order set by
//     (M, N, K, G)), with no floating-point atomics.
//
// Inside a segment: a tile is RB row blocks (16 rows each) x one m tile.  The segment's chunk
// range is cut into 16 contiguous sub-ranges, one per (wave w, lane group g) pair; lane
// (r = lane % 16, g = lane / 16) of wave w handles row r of every row block of the tile on
// sub-range 4w + g, so the X values it loads serve RB row blocks.
#include <mutex>

#include "w12_device.h"
#include "w12_kernels.h"

namespace w12 {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kSubRanges = kWaves * 4;
constexpr int kUnitChunks = kSubRanges;   // chunks per stream-K unit (one per sub-range)
constexpr int kRB = 4;                    // row blocks per tile (64 rows)
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past any plane: reads give 0

__device__ __forceinline__ int64_t split_point(int64_t total, int64_t parts, int64_t q) { return q * total / parts; }
__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct GemmArgs {
  const uint16_t* X;
  int64_t ldx;
  const uint8_t* base;
  const uint8_t* hi;
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc;
  uint32_t num_esc;
  int32_t M, N, K;
  int64_t Kc, Nb;
  int32_t MT;           // m tiles
  int64_t tiles;        // row groups x m tiles
  int64_t upt;          // units per tile
  int64_t units;        // tiles x upt
  int64_t G;            // work-groups
  uint32_t hi_bytes, lo_bytes, x_bytes;
  float* Y;
  int64_t ldy;
  uint32_t* counters;   // [tiles]
  float* P;             // [2G][tile elements]
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
// 16 bytes per lane from the buffer into LDS: lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, 0, 0, 0);
}

// ------------------------------------------------------------------------------------------
// Reading the ring.  The compiler's waits for buffer-to-LDS loads model each DMA as a 16-byte
// write at its base address (the wave actually writes 16 bytes per lane), so it can miss a
// dependency or wait for far more than needed.  The ring is therefore read with explicit
// instructions the compiler does not associate with the DMA, after an explicit vmcnt wait
// for the stage: all other memory traffic stays under the compiler's own accounting.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)(lds_u8*)p; }

// Wait until at most N vector-memory instructions of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// One stage's LDS reads and the wait for them in a single statement, so no register holding
// a value still in flight is ever visible to the compiler.  Outputs are early-clobber: they
// are written while later reads of the statement still use the address inputs.
#define W12_W_READS                                                                          \
  "ds_read_b128 %0, %[ah] offset:0\n"                                                        \
  "ds_read_b128 %1, %[ah] offset:1024\n"                                                     \
  "ds_read_b128 %2, %[ah] offset:2048\n"                                                     \
  "ds_read_b128 %3, %[ah] offset:3072\n"                                                     \
  "ds_read_b64 %4, %[al] offset:0\n"                                                         \
  "ds_read_b64 %5, %[al] offset:512\n"                                                       \
  "ds_read_b64 %6, %[al] offset:1024\n"                                                      \
  "ds_read_b64 %7, %[al] offset:1536\n"
#define W12_W_OUTS(h, l)                                                                     \
  "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(l[0]), "=&v"(l[1]), "=&v"(l[2]), "=&v"(l[3])

__device__ __forceinline__ void read_stage_w(uint32_t ah, uint32_t al, uint4 h[4], uint2 l[4]) {
  asm volatile(W12_W_READS "s_waitcnt lgkmcnt(0)"
               : W12_W_OUTS(h, l)
               : [ah] "v"(ah), [al] "v"(al)
               : "memory");
}

// The W reads plus X rows 0..M-1 (two 16-byte pieces each, 128 bytes apart per row).
#define W12_X2(i, off) "ds_read_b128 %" #i ", %[ax] offset:" #off "\n"
template <int M>
__device__ __forceinline__ void read_stage_wx(uint32_t ah, uint32_t al, uint32_t ax, uint4 h[4], uint2 l[4],
                                              uint4 xa[M], uint4 xb[M]) {
  static_assert(M >= 1 && M <= 8, "GEMV rows");
  if constexpr (M == 1) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else if constexpr (M == 2) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 128) W12_X2(11, 144) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else if constexpr (M == 3) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 128) W12_X2(11, 144) W12_X2(12, 256)
                     W12_X2(13, 272) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1]), "=&v"(xa[2]),
                   "=&v"(xb[2])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else if constexpr (M == 4) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 128) W12_X2(11, 144) W12_X2(12, 256)
                     W12_X2(13, 272) W12_X2(14, 384) W12_X2(15, 400) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1]), "=&v"(xa[2]),
                   "=&v"(xb[2]), "=&v"(xa[3]), "=&v"(xb[3])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else {
    // M = 5..8: rows 0-3 with the W reads, rows 4..M-1 in a second statement
    read_stage_wx<4>(ah, al, ax, h, l, xa, xb);
    if constexpr (M == 5) {
      asm volatile(W12_X2(0, 512) W12_X2(1, 528) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(xa[4]), "=&v"(xb[4]) : [ax] "v"(ax) : "memory");
    } else if constexpr (M == 6) {
      asm volatile(W12_X2(0, 512) W12_X2(1, 528) W12_X2(2, 640) W12_X2(3, 656) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(xa[4]), "=&v"(xb[4]), "=&v"(xa[5]), "=&v"(xb[5]) : [ax] "v"(ax) : "memory");
    } else if constexpr (M == 7) {
      asm volatile(W12_X2(0, 512) W12_X2(1, 528) W12_X2(2, 640) W12_X2(3, 656) W12_X2(4, 768) W12_X2(5, 784)
                       "s_waitcnt lgkmcnt(0)"
                   : "=&v"(xa[4]), "=&v"(xb[4]), "=&v"(xa[5]), "=&v"(xb[5]), "=&v"(xa[6]), "=&v"(xb[6])
                   : [ax] "v"(ax) : "memory");
    } else {
      asm volatile(W12_X2(0, 512) W12_X2(1, 528) W12_X2(2, 640) W12_X2(3, 656) W12_X2(4, 768) W12_X2(5, 784)
                       W12_X2(6, 896) W12_X2(7, 912) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(xa[4]), "=&v"(xb[4]), "=&v"(xa[5]), "=&v"(xb[5]), "=&v"(xa[6]), "=&v"(xb[6]),
                     "=&v"(xa[7]), "=&v"(xb[7])
                   : [ax] "v"(ax) : "memory");
    }
  }
}

// ------------------------------------------------------------------------------------------
// Escapes: per lane and row block, a cursor over the channel's entries with k >= the start of
// the lane's range.  Entries past the range are never reached (their k is beyond every chunk
// the lane decodes), so the cursor needs no end of range.
// ------------------------------------------------------------------------------------------
struct LaneEsc {
  uint32_t pos, end;   // next entry and end of the channel's list
  uint32_t e;          // the entry at pos (valid when pos < end)
};

__device__ __forceinline__ void esc_start(LaneEsc& c, const GemmArgs& g, int64_t n, uint32_t k_lo) {
  c.pos = c.end = 0;
  c.e = 0;
  if (n >= g.N) return;
  uint32_t e_lo, e_hi;
  escape_range(g.esc_ptr, n, g.num_esc, e_lo, e_hi);
  const uint32_t cnt = e_hi - e_lo;
  if (cnt == 0) return;
  if (cnt <= 4) {
    // the common case (about one escape per 5120 weights): four independent loads
    uint32_t v[4], skip = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ((uint32_t)i < cnt) ? g.esc[e_lo + i] : 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) skip += ((uint32_t)i < cnt) && ((v[i] >> 16) < k_lo);
    c.pos = e_lo + skip;
    c.end = e_hi;
    c.e = skip == 0 ? v[0] : (skip == 1 ? v[1] : (skip == 2 ? v[2] : v[3]));
  } else {
    c.pos = lower_bound_k(g.esc, e_lo, e_hi, k_lo);
    c.end = e_hi;
    c.e = c.pos < c.end ? g.esc[c.pos] : 0u;
  }
}

// Patch every escape of this lane's row that falls in chunk [k0, k0 + 16).
__device__ __forceinline__ void esc_apply(LaneEsc& c, const uint32_t* __restrict__ esc, uint32_t k0, uint32_t d[8]) {
  while (c.pos < c.end && (c.e >> 16) < k0 + kChunkK) {
    patch16(d, (c.e >> 16) - k0, c.e & 0xFFFFu);
    ++c.pos;
    c.e = c.pos < c.end ? esc[c.pos] : 0u;
  }
}

// ------------------------------------------------------------------------------------------
// LDS ring (per work-group; each wave owns its slice).  One object per stage lets the
// compiler wait for exactly the stage being read.
// ------------------------------------------------------------------------------------------
template <int RB>
struct RingStage {
  uint4 hi[kWaves][RB][kWave];        // lane (r, g): its 16 hi bytes of row block rb
  uint4 lo[kWaves][RB * 32];          // [rb][g][16 rows x 8 bytes]
};

// Per-lane addressing of one segment.
struct SegLane {
  uint32_t c_lo, c_hi, iters;   // this lane's chunks [c_lo, c_hi) (may be empty); iterations
  uint32_t c_at;                // an in-range chunk to read when past the range
  uint32_t cd_lo, cd_hi, cd_at; // the same for lane group (lane >> 3) & 3 (lo DMA)
  uint32_t lo_rb0, lo_rb1;      // lo plane offsets of the row blocks this lane DMAs
};

template <int RB>
__device__ __forceinline__ void issue_w(const GemmArgs& g, __amdgpu_buffer_rsrc_t rh, __amdgpu_buffer_rsrc_t rl,
                                        const uint32_t soff_h[RB], const SegLane& sl, uint32_t j,
                                        RingStage<RB>* st, int wave) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const uint32_t c = (sl.c_lo + j < sl.c_hi) ? sl.c_lo + j : sl.c_at;   // past the range: unused re-read
  const uint32_t vh = (c * kRowsPerBlock + r) * kChunkK;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void*)&st->hi[wave][rb][0], 16, (int)vh, (int)soff_h[rb], 0, 0);
  const uint32_t cd = (sl.cd_lo + j < sl.cd_hi) ? sl.cd_lo + j : sl.cd_at;
  const uint32_t vl = cd * kLoChunkBytes + (lane & 7) * 16;
  dma16(rl, &st->lo[wave][0], sl.lo_rb0 + vl);
  if (RB > 2) dma16(rl, &st->lo[wave][64], sl.lo_rb1 + vl);
}

// Byte addresses (in LDS) of this lane's hi and lo slots of row block 0 of a stage.
template <int RB>
__device__ __forceinline__ void ring_addr(const RingStage<RB>* st, int wave, uint32_t& ah, uint32_t& al) {
  const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
  ah = lds_off(&st->hi[wave][0][lane]);
  al = lds_off(&st->lo[wave][0]) + gq * 128 + r * 8;
}

// ------------------------------------------------------------------------------------------
// The two inner products.
// ------------------------------------------------------------------------------------------
// M <= 8 (wavefront GEMV): every lane needs all M rows of X at its chunk; the wave's 4M
// (row, chunk) X pieces ride the LDS ring and are read back as broadcasts.
template <int M>
struct GemvPath {
  static constexpr int kMRows = M;
  static constexpr bool kXInLds = true;
  static constexpr int kVmemPerStage = 7;   // 6 W DMA + 1 X DMA
  typedef float Acc;
  static constexpr int kAcc = M;
  struct XStage {
    uint4 x[kWaves][kWave];   // [m][g][half]
  };
  // lanes l < 8M fetch (m = l / 8, lane group l / 2 % 4, half l % 2)
  __device__ static void issue_x(const GemmArgs& g, __amdgpu_buffer_rsrc_t rx, const uint32_t xc_lo,
                                 const uint32_t xc_hi, uint32_t j, XStage* xs, int wave) {
    const int lane = threadIdx.x & 63;
    const uint32_t m = (uint32_t)lane >> 3, half = lane & 1;
    const uint32_t c = xc_lo + j;
    const uint32_t off = (m < (uint32_t)M && c < xc_hi) ? (m * (uint32_t)g.ldx + c * kChunkK) * 2u + half * 16u
                                                        : kOutOfRange;
    dma16(rx, &xs->x[wave][0], off);
  }
  __device__ static void zero(Acc acc[]) {
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
  }
  // this lane's X pieces (its lane group's chunk, all M rows) of a stage
  __device__ static uint32_t x_addr(const XStage* xs, int wave) {
    const int gq = (threadIdx.x & 63) >> 4;
    return lds_off(&xs->x[wave][gq * 2]);
  }
  __device__ static void mac(const uint32_t d[8], const uint4 xa[M], const uint4 xb[M], Acc acc[]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t xv[8] = {xa[m].x, xa[m].y, xa[m].z, xa[m].w, xb[m].x, xb[m].y, xb[m].z, xb[m].w};
#pragma unroll
      for (int p = 0; p < 8; ++p)
        acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[p]), __builtin_bit_cast(bf16x2, xv[p]),
                                                 acc[m], false);
    }
  }
  // Reduce over the 4 lane groups with a fixed butterfly, then add this wave's values into
  // red[row][m] (waves in order 0..3, called once per wave in that order).
  __device__ static void to_lds(Acc acc[], int rb, float* red, bool first_wave) {
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[m];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[m] = v;
    }
    if (gq == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float* dst = &red[(rb * kRowsPerBlock + r) * M + m];
        *dst = first_wave ? acc[m] : *dst + acc[m];
      }
    }
  }
};

// M >= 9: MB m blocks of 16 rows; lane (r, g) supplies X row m0 + 16 mb + r of its own chunk,
// loaded one iteration ahead into registers.
template <int MB>
struct MfmaPath {
  static constexpr int kMRows = MB * 16;
  static constexpr bool kXInLds = false;
  static constexpr int kVmemPerStage = 6 + 2 * MB;   // 6 W DMA + X loads
  typedef f32x4 Acc;
  static constexpr int kAcc = MB;
  struct XStage {};
  __device__ static void load_x(const GemmArgs& g, __amdgpu_buffer_rsrc_t rx, int m0, uint32_t c, bool ok, uint4 xa[MB],
                                uint4 xb[MB]) {
    const int r = threadIdx.x & 15;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint32_t m = (uint32_t)(m0 + mb * 16 + r);
      const uint32_t off = (ok && m < (uint32_t)g.M) ? (m * (uint32_t)g.ldx + c * kChunkK) * 2u : kOutOfRange;
      xa[mb] = bload16(rx, off);
      xb[mb] = bload16(rx, off + 16);
    }
  }
  __device__ static void zero(Acc acc[]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ static void mac(const uint32_t d[8], const uint4 xa[MB], const uint4 xb[MB], Acc acc[]) {
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(d[4], d[5], d[6], d[7]));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mb]), b0, acc[mb], 0, 0, 0);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xb[mb]), b1, acc[mb], 0, 0, 0);
    }
  }
  // lane (r, g) holds C[m = 4g + i][n = r] of each m block
  __device__ static void to_lds(Acc acc[], int rb, float* red, bool first_wave) {
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* dst = &red[(rb * kRowsPerBlock + r) * kMRows + mb * 16 + 4 * gq + i];
        *dst = first_wave ? acc[mb][i] : *dst + acc[mb][i];
      }
  }
};

// ------------------------------------------------------------------------------------------
// Segment epilogue.  Cross-work-group visibility without cache-wide fences: the segments of
// a tile may run on different XCDs, whose L2 caches are not coherent with each other.  Every
// access to the partial buffer and to the arrival counter is a device-scope (agent) atomic
// access, performed at the device coherence point (stores and loads carry sc1, the counter
// RMW is device-coherent), and each wave waits for its partial stores to complete
// (vmcnt(0)) before the barrier that precedes the counter increment.  Agent-scope
// release/acquire fences would write back / invalidate the whole L2 of the XCD instead.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0xF70); /* vmcnt(0) */ }

// Stream-K bookkeeping: work-group w owns units [ubeg(w), ubeg(w+1)).
__device__ __forceinline__ int64_t ubeg(const GemmArgs& g, int64_t w) { return w * g.units / g.G; }

template <int ROWS, int MROWS>
__device__ __forceinline__ void finish_segment(const GemmArgs& g, const float* red, int64_t tile, int64_t rg, int m0,
                                               bool full, bool first_seg, uint32_t* s_flag) {
  const int64_t n0 = rg * ROWS;
  if (full) {
    for (int i = threadIdx.x; i < ROWS * MROWS; i += kThreads) {
      const int row = i / MROWS, ml = i % MROWS;
      const int64_t n = n0 + row;
      const int m = m0 + ml;
      if (n < g.N && m < g.M) g.Y[(int64_t)m * g.ldy + n] = red[i];
    }
    return;
  }
  const int64_t w = blockIdx.x;
  float* mine = g.P + (2 * w + (first_seg ? 0 : 1)) * (int64_t)(ROWS * MROWS);
  for (int i = threadIdx.x; i < ROWS * MROWS; i += kThreads)
    __hip_atomic_store(mine + i, red[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_vm_all();
  // segments of this tile: work-groups w_a..w_b
  const int64_t t0 = tile * g.upt;
  const int64_t w_a = ceil_div((t0 + 1) * g.G, g.units) - 1;
  const int64_t w_b = ceil_div((t0 + g.upt) * g.G, g.units) - 1;
  const uint32_t nseg = (uint32_t)(w_b - w_a + 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(g.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == nseg - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (*s_flag == 0) return;
  for (int i = threadIdx.x; i < ROWS * MROWS; i += kThreads) {
    const int row = i / MROWS, ml = i % MROWS;
    const int64_t n = n0 + row;
    const int m = m0 + ml;
    float v = 0.f;
    for (int64_t wj = w_a; wj <= w_b; ++wj) {
      const int pos = ubeg(g, wj) >= t0 ? 0 : 1;   // the tile's segment is wj's first, else its last
      const float p = __hip_atomic_load(g.P + (2 * wj + pos) * (int64_t)(ROWS * MROWS) + i, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      v = (wj == w_a) ? p : v + p;
    }
    if (n < g.N && m < g.M) g.Y[(int64_t)m * g.ldy + n] = v;
  }
  if (threadIdx.x == 0) __hip_atomic_store(g.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------------
// The kernel.
// ------------------------------------------------------------------------------------------
template <class Path>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs g) {
  constexpr int RB = kRB;
  constexpr int ROWS = RB * kRowsPerBlock;
  constexpr int MROWS = Path::kMRows;
  typedef typename Path::XStage XStage;
  __shared__ RingStage<RB> ring0, ring1;
  __shared__ XStage xring0, xring1;
  __shared__ uint32_t s_flag;
  static_assert(sizeof(RingStage<RB>) >= ROWS * MROWS * sizeof(float), "reduction buffer aliases stage 0");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, gq = lane >> 4;
  const int q = wave * 4 + gq;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(g.hi, g.hi_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(g.lo, g.lo_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.X, g.x_bytes);

  int64_t u = ubeg(g, blockIdx.x);
  const int64_t u_first = u;
  const int64_t u_end = ubeg(g, (int64_t)blockIdx.x + 1);
  while (u < u_end) {
    const int64_t tile = u / g.upt;
    const int64_t t0 = tile * g.upt;
    const int64_t seg_end = u_end < t0 + g.upt ? u_end : t0 + g.upt;
    const int64_t rg = tile / g.MT;
    const int m0 = (int)(tile % g.MT) * MROWS;
    // this segment's chunks [cs0, cs1) and this lane's sub-range of them
    const int64_t cs0 = (u - t0) * kUnitChunks;
    const int64_t cs1 = ((seg_end - t0) * kUnitChunks < g.Kc) ? (seg_end - t0) * kUnitChunks : g.Kc;
    SegLane sl;
    sl.c_lo = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, q));
    sl.c_hi = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, q + 1));
    sl.iters = (uint32_t)ceil_div(cs1 - cs0, kSubRanges);
    const int qd = wave * 4 + ((lane >> 3) & 3);
    sl.cd_lo = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qd));
    sl.cd_hi = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qd + 1));
    // past its range (or for an empty range) a lane re-reads an in-range chunk, unused
    sl.c_at = sl.c_lo < (uint32_t)g.Kc ? sl.c_lo : (uint32_t)g.Kc - 1;
    sl.cd_at = sl.cd_lo < (uint32_t)g.Kc ? sl.cd_lo : (uint32_t)g.Kc - 1;
    const int64_t row0 = rg * ROWS;
    uint32_t soff_h[RB], bb2[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      int64_t rbg = rg * RB + rb;
      rbg = rbg < g.Nb ? rbg : g.Nb - 1;   // a ragged last tile re-reads its last row block
      soff_h[rb] = (uint32_t)(rbg * g.Kc * kHiChunkBytes);
      const int64_t n = row0 + rb * kRowsPerBlock + r;
      bb2[rb] = base_pair(n < g.N ? g.base[n] : 1u);
    }
    {
      int64_t rb0 = rg * RB + (lane >> 5), rb1 = rg * RB + 2 + (lane >> 5);
      rb0 = rb0 < g.Nb ? rb0 : g.Nb - 1;
      rb1 = rb1 < g.Nb ? rb1 : g.Nb - 1;
      sl.lo_rb0 = (uint32_t)(rb0 * g.Kc * kLoChunkBytes);
      sl.lo_rb1 = (uint32_t)(rb1 * g.Kc * kLoChunkBytes);
    }
    // X chunk range of the lane group this lane fetches X for (GEMV: lane / 2 % 4)
    const int qx = wave * 4 + ((lane >> 1) & 3);
    const uint32_t xc_lo = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qx));
    const uint32_t xc_hi = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qx + 1));

    // escape cursors first (their loads retire before the DMA issued after them)
    LaneEsc cur[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) esc_start(cur[rb], g, row0 + rb * kRowsPerBlock + r, sl.c_lo * kChunkK);

    // stage 0 (and X 0) in flight
    issue_w<RB>(g, rh, rl, soff_h, sl, 0, &ring0, wave);
    uint4 xa0[Path::kAcc], xb0[Path::kAcc], xa1[Path::kAcc], xb1[Path::kAcc];
    if constexpr (Path::kXInLds) {
      Path::issue_x(g, rx, xc_lo, xc_hi, 0, &xring0, wave);
    } else {
      Path::load_x(g, rx, m0, sl.c_lo, sl.c_lo < sl.c_hi, xa0, xb0);
    }
    typename Path::Acc acc[RB][Path::kAcc];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) Path::zero(acc[rb]);

    uint32_t ah0, al0, ah1, al1;
    ring_addr<RB>(&ring0, wave, ah0, al0);
    ring_addr<RB>(&ring1, wave, ah1, al1);
    // stage j is complete once at most `pending` newer vector-memory instructions remain
    auto compute = [&](uint32_t ah, uint32_t al, const XStage* xs, uint4* xa, uint4* xb, uint32_t j, bool pending) {
      if (pending) wait_vmcnt<Path::kVmemPerStage>();
      else wait_vmcnt<0>();
      static_assert(RB == 4, "ring reads are written for 4 row blocks");
      uint4 h[RB];
      uint2 l[RB];
      if constexpr (Path::kXInLds) read_stage_wx<Path::kAcc>(ah, al, Path::x_addr(xs, wave), h, l, xa, xb);
      else read_stage_w(ah, al, h, l);
      const uint32_t c = sl.c_lo + j;
      const bool valid = c < sl.c_hi;
      const uint32_t k0 = c * kChunkK;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t d[8];
        decode16(h[rb], l[rb], bb2[rb], d);
        if (valid) esc_apply(cur[rb], g.esc, k0, d);
        Path::mac(d, xa, xb, acc[rb]);
      }
    };
    for (uint32_t j = 0; j < sl.iters; j += 2) {
      const bool more1 = j + 1 < sl.iters;
      if (more1) {
        issue_w<RB>(g, rh, rl, soff_h, sl, j + 1, &ring1, wave);
        if constexpr (Path::kXInLds) Path::issue_x(g, rx, xc_lo, xc_hi, j + 1, &xring1, wave);
        else Path::load_x(g, rx, m0, sl.c_lo + j + 1, sl.c_lo + j + 1 < sl.c_hi, xa1, xb1);
      }
      compute(ah0, al0, &xring0, xa0, xb0, j, more1);
      if (!more1) break;
      const bool more2 = j + 2 < sl.iters;
      if (more2) {
        issue_w<RB>(g, rh, rl, soff_h, sl, j + 2, &ring0, wave);
        if constexpr (Path::kXInLds) Path::issue_x(g, rx, xc_lo, xc_hi, j + 2, &xring0, wave);
        else Path::load_x(g, rx, m0, sl.c_lo + j + 2, sl.c_lo + j + 2 < sl.c_hi, xa0, xb0);
      }
      compute(ah1, al1, &xring1, xa1, xb1, j + 1, more2);
    }
    __syncthreads();   // every wave is done with the ring; stage 0 becomes the reduction buffer
    float* red = reinterpret_cast<float*>(&ring0);
    for (int w = 0; w < kWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) Path::to_lds(acc[rb], rb, red, w == 0);
      }
      __syncthreads();
    }
    const bool full = (u == t0) && (seg_end == t0 + g.upt);
    finish_segment<ROWS, MROWS>(g, red, tile, rg, m0, full, u == u_first, &s_flag);
    __syncthreads();   // LDS is reused by the next segment
    u = seg_end;
  }
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The ragged-K GEMM (K not a multiple of 16) reads X element by element; it is a separate,
// simpler kernel: X is first copied into a zero-padded [M][Kc * 16] buffer in the workspace.
__global__ __launch_bounds__(256) void k_pad_x(const uint16_t* __restrict__ X, int64_t ldx, int32_t M, int32_t K,
                                               int64_t kp, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * kp) return;
  const int64_t m = i / kp, k = i % kp;
  out[i] = k < K ? X[m * ldx + k] : (uint16_t)0;
}

// ------------------------------------------------------------------------------------------
// Planning and launch
// ------------------------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}

// Compute units of the current device (256 on MI355X; that value is also used when no device
// is visible, so host-only planning gives the same sizes as on the GPU).
static int device_cus() {
  static std::once_flag once;
  static int cus = 256;
  std::call_once(once, [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      (void)hipGetLastError();
  });
  return cus;
}

template <class Path>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs g);

// Resident work-groups per CU of one kernel variant, from the runtime occupancy calculator
// (registers and LDS of the compiled kernel); when no device is visible, a conservative
// estimate.  Cached per variant.
template <class Path>
static int occupancy_of(int fallback) {
  static std::once_flag once;
  static int v = 0;
  std::call_once(once, [fallback] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&k_gemm<Path>), kThreads, 0) ==
            hipSuccess && n > 0)
      v = n;
    else {
      (void)hipGetLastError();
      v = fallback;
    }
  });
  return v;
}

template <int M>
struct GemvPath;
template <int MB>
struct MfmaPath;

static int groups_per_cu(int path, int M, int m_tile) {
  if (path == 1) {
    switch (M) {
      case 1: return occupancy_of<GemvPath<1>>(2);
      case 2: return occupancy_of<GemvPath<2>>(2);
      case 3: return occupancy_of<GemvPath<3>>(2);
      case 4: return occupancy_of<GemvPath<4>>(2);
      case 5: return occupancy_of<GemvPath<5>>(2);
      case 6: return occupancy_of<GemvPath<6>>(2);
      case 7: return occupancy_of<GemvPath<7>>(2);
      default: return occupancy_of<GemvPath<8>>(2);
    }
  }
  switch (m_tile / 16) {
    case 1: return occupancy_of<MfmaPath<1>>(3);
    case 2: return occupancy_of<MfmaPath<2>>(2);
    case 3: return occupancy_of<MfmaPath<3>>(1);
    default: return occupancy_of<MfmaPath<4>>(1);
  }
}

GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K) {
  GemmPlan p{};
  p.path = (M <= 8) ? 1 : 2;
  p.rb = kRB;
  p.waves = kWaves;
  const int64_t Nb = num_row_blocks(N);
  const int64_t Kc = num_chunks(K);
  p.row_groups = (Nb + p.rb - 1) / p.rb;
  if (p.path == 1) {
    p.m_tile = M;
    p.m_tiles = 1;
  } else {
    const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 48 ? 3 : 4));
    p.m_tile = 16 * mb;
    p.m_tiles = (M + p.m_tile - 1) / p.m_tile;
  }
  p.tiles = p.row_groups * p.m_tiles;
  p.upt = (Kc + kUnitChunks - 1) / kUnitChunks;
  p.units = p.tiles * p.upt;
  int64_t G = (int64_t)device_cus() * env_int("W12_GROUPS_PER_CU", groups_per_cu(p.path, M, p.m_tile));
  if (G > p.units) G = p.units;
  if (G < 1) G = 1;
  p.grid = G;
  // segments per tile (1 when every work-group covers whole tiles)
  p.splits = (int)((p.upt * G + p.units - 1) / p.units);
  if (p.splits < 1) p.splits = 1;
  const uint64_t tile_elems = (uint64_t)p.rb * kRowsPerBlock * (uint64_t)p.m_tile;
  p.counter_bytes = ((uint64_t)p.tiles * 4 + 255) / 256 * 256;
  p.partial_bytes = 2ull * (uint64_t)G * tile_elems * sizeof(float);
  // ragged K: room for X padded to whole chunks
  p.xpad_bytes = (K % kChunkK) ? ((uint64_t)M * (uint64_t)Kc * kChunkK * 2 + 255) / 256 * 256 : 0;
  p.ws_bytes = p.counter_bytes + p.partial_bytes + p.xpad_bytes;
  return p;
}

template <class Path>
static void launch_path(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm<Path>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
}

static void dispatch(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  if (p.path == 1) {
    switch (a.M) {
      case 1: launch_path<GemvPath<1>>(p, a, stream); break;
      case 2: launch_path<GemvPath<2>>(p, a, stream); break;
      case 3: launch_path<GemvPath<3>>(p, a, stream); break;
      case 4: launch_path<GemvPath<4>>(p, a, stream); break;
      case 5: launch_path<GemvPath<5>>(p, a, stream); break;
      case 6: launch_path<GemvPath<6>>(p, a, stream); break;
      case 7: launch_path<GemvPath<7>>(p, a, stream); break;
      default: launch_path<GemvPath<8>>(p, a, stream); break;
    }
  } else {
    switch (p.m_tile / 16) {
      case 1: launch_path<MfmaPath<1>>(p, a, stream); break;
      case 2: launch_path<MfmaPath<2>>(p, a, stream); break;
      case 3: launch_path<MfmaPath<3>>(p, a, stream); break;
      default: launch_path<MfmaPath<4>>(p, a, stream); break;
    }
  }
}

hipError_t init_gemm_workspace(void* ws, uint64_t bytes, hipStream_t stream) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(ws), words);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y,
                       int64_t ldy, void* ws, hipStream_t stream) {
  GemmArgs a;
  a.Kc = num_chunks(t->K);
  if (p.xpad_bytes) {
    // ragged K: copy X into whole zero-padded chunks first
    uint16_t* xp = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes + p.partial_bytes);
    const int64_t kp = a.Kc * kChunkK;
    const int64_t total = (int64_t)M * kp;
    hipLaunchKernelGGL(k_pad_x, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, X, ldx, M, t->K, kp, xp);
    X = xp;
    ldx = kp;
  }
  a.X = X;
  a.ldx = ldx;
  a.base = t->base;
  a.hi = t->hi;
  a.lo = t->lo;
  a.esc_ptr = t->esc_ptr;
  a.esc = t->esc;
  a.num_esc = (uint32_t)t->num_escapes;
  a.M = M;
  a.N = t->N;
  a.K = t->K;
  a.Nb = num_row_blocks(t->N);
  a.MT = p.m_tiles;
  a.tiles = p.tiles;
  a.upt = p.upt;
  a.units = p.units;
  a.G = p.grid;
  const uint64_t chunks = (uint64_t)a.Nb * (uint64_t)a.Kc;
  a.hi_bytes = (uint32_t)(chunks * kHiChunkBytes);
  a.lo_bytes = (uint32_t)(chunks * kLoChunkBytes);
  a.x_bytes = (uint32_t)(((uint64_t)(M - 1) * (uint64_t)ldx + (uint64_t)a.Kc * kChunkK) * 2u);
  a.Y = Y;
  a.ldy = ldy;
  a.counters = reinterpret_cast<uint32_t*>(ws);
  a.P = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes);
  dispatch(p, a, stream);
  return hipGetLastError();
}

}  // namespace w12
