// W12 GEMM: Y[M][N] = X[M][K] . W[N][K]^T with BF16 X, W12 weights and FP32 accumulation.
//
// What the GEMM must do is set by the SpecPilot summary page, method bullet of section 4.1:
// decode W12 records in registers inside a stream-K GEMM, and reduce the K split in an order
// fixed in advance, so repeated runs give identical bits.  This gfx950 version:
//   * streams the hi/lo record planes from HBM into a per-wave LDS ring (two stages; three for
//     the 64-row tiles) with non-temporal buffer-to-LDS DMA loads (no registers held while a
//     stage is in flight; the planes are read once and stream through L2), reads each
//     lane's 16 + 8 bytes back, decodes them to BF16 pairs in registers (decode16) and
//     patches the escapes of the lane's chunk from its channel's escape list, which sits in
//     LDS (copied one segment ahead); tensors whose lists do not fit there on average run an
//     instantiation of their own that reads them from global memory through register windows
//     (EscWin);
//   * small M (the wavefront GEMV): FP32 dot2 (v_dot2c_f32_bf16) accumulation per lane, a
//     fixed butterfly over the 4 lane groups and a fixed wave order through LDS; X rides the
//     ring;
//   * larger M: the decoded chunk is the B operand of v_mfma_f32_16x16x32_bf16 (16 rows of W x
//     32 k) and X rows (padded to 16) are the A operand, staged in the LDS ring beside the
//     records (16, 48 and 64 rows) or double-buffered in registers (32 rows);
//   * schedules work stream-K style: the grid is at most the number of work-groups resident at
//     once, and work-group w (its logical index, laid out per XCD) takes the contiguous range
//     [w U / G, (w+1) U / G) of the U = tiles x units work units (a unit is 16 chunks of one
//     tile), so every work-group streams the same number of bytes.  A tile covered by several work-groups gets one partial per
//     segment; the last segment to finish sums them in segment order (a fixed order set by
//     (M, N, K, G)), with no floating-point atomics.
//
// Inside a segment: a tile is RB row blocks (16 rows each) x one m tile.  Lane (r = lane % 16,
// g = lane / 16) of wave w belongs to lane group q = 4 w + g and handles row r of every row
// block of the tile on the chunks of lane group q, so the X values it loads serve RB row
// blocks.
#include <mutex>
#include <type_traits>
#include <vector>

#include "w12_device.h"
#include "w12_gemm_common.h"
#include "w12_kernels.h"

namespace w12 {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kSubRanges = kWaves * 4;
constexpr int kUnitChunks = kSubRanges;   // chunks per stream-K unit (one per sub-range)
constexpr int kRB = 4;                    // row blocks per tile (64 rows)
constexpr int kTileRows = kRB * kRowsPerBlock;

__device__ __forceinline__ int64_t split_point(int64_t total, int64_t parts, int64_t q) { return q * total / parts; }

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
  int64_t ubase;        // first unit of this product in the launch's unit space (0 unless grouped)
  int64_t units;        // units of the whole launch (every product of a group)
  int64_t G;            // work-groups
  uint32_t hi_bytes, lo_bytes, x_bytes, esc_bytes, y_bytes, p_bytes;
  float* Y;
  int64_t ldy;
  uint32_t* counters;   // [kMaxGrid] arrival counters, indexed by a split tile's first work-group
  float* P;             // [2G][tile elements] partial tiles (shared by a group)
};

// Several independent products of one launch (same M): work-group w takes units
// [w U / G, (w+1) U / G) of their concatenated unit spaces, product i owning
// [g[i].ubase, g[i].ubase + g[i].tiles * g[i].upt).  A single product is a group of one.
constexpr int kGroupMax = 8;
template <int NG>
struct GroupArgs {
  GemmArgs g[NG];
  int32_t count;
};

// More products than the kernel arguments hold (whole models in one launch): their arguments
// sit in device memory, in the workspace after the partial tiles, in launch order.
struct GroupArgsDev {
  const GemmArgs* g;
  int32_t count;
};
// The argument block of a launch: NG products in the kernel arguments, or (NG = 0) any number
// in device memory.
template <int NG>
struct ArgsOf {
  typedef GroupArgs<NG> type;
};
template <>
struct ArgsOf<0> {
  typedef GroupArgsDev type;
};

// Product i's argument block.  Device-memory blocks are read through the constant address
// space (nothing writes them during the launch), as kernel arguments are: their loads stay
// scalar, and the pointers loaded from them stay global (flat loads would also count on the LDS
// wait counter).
template <int NG, class I>
__device__ __forceinline__ const GemmArgs& arg_at(const GroupArgs<NG>& ga, I i) {
  return ga.g[i];
}
template <class I>
__device__ __forceinline__ const GemmArgs& arg_at(const GroupArgsDev& ga, I i) {
  typedef const __attribute__((address_space(4))) GemmArgs ConstArgs;
  ConstArgs* p = (ConstArgs*)(uintptr_t)ga.g;
  return *(const GemmArgs*)(p + i);
}

// The product that owns unit u (uniform).
template <int NG>
__device__ __forceinline__ int gemm_of(const GroupArgs<NG>& ga, int64_t u) {
  int gi = 0;
  if constexpr (NG > 1) {
#pragma unroll
    for (int i = 1; i < NG; ++i)
      if (i < ga.count && u >= ga.g[i].ubase) gi = i;
  }
  return gi;
}
__device__ __forceinline__ int gemm_of(const GroupArgsDev& ga, int64_t u) {
  int lo = 0, hi = ga.count - 1;   // the last product whose first unit is <= u
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (arg_at(ga, mid).ubase <= u) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// The product that owns unit u, given that product gi owns an earlier unit (uniform).
template <int NG>
__device__ __forceinline__ int gemm_from(const GroupArgs<NG>& ga, int gi, int64_t u) {
  (void)gi;
  return gemm_of(ga, u);
}
__device__ __forceinline__ int gemm_from(const GroupArgsDev& ga, int gi, int64_t u) {
  while (gi + 1 < ga.count && arg_at(ga, gi + 1).ubase <= u) ++gi;
  return gi;
}

// Buffer resources of one product's operands.
struct Res {
  __amdgpu_buffer_rsrc_t h, l, x, p, e, base, y;
};
__device__ __forceinline__ Res make_res(const GemmArgs& g) {
  Res r;
  r.h = make_rsrc(g.hi, g.hi_bytes);
  r.l = make_rsrc(g.lo, g.lo_bytes);
  r.x = make_rsrc(g.X, g.x_bytes);
  r.p = make_rsrc(g.esc_ptr, (uint32_t)(g.N + 1) * 4u);
  r.e = make_rsrc(g.esc, g.esc_bytes);
  r.base = make_rsrc(g.base, (uint32_t)g.N);
  r.y = make_rsrc(g.Y, g.y_bytes);
  return r;
}

// ------------------------------------------------------------------------------------------
// Reading the ring.  The compiler's waits for buffer-to-LDS loads model each DMA as a 16-byte
// write at its base address (the wave actually writes 16 bytes per lane), so it can miss a
// dependency or wait for far more than needed.  The ring is therefore read with explicit
// instructions the compiler does not associate with the DMA, after an explicit vmcnt wait
// for the stage: all other memory traffic stays under the compiler's own accounting.
// ------------------------------------------------------------------------------------------
// Batched LDS reads with literal offsets, one statement and one wait each (no register still
// in flight is ever visible to the compiler).
// M dwords 256 bytes apart (GEMV partials: one channel, M rows of X, red laid out [m][64]).
template <int M>
__device__ __forceinline__ void lds_read_m(uint32_t a, uint32_t o[M]) {
  if constexpr (M == 1) {
    asm volatile("ds_read_b32 %0, %1 offset:0\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]) : "v"(a) : "memory");
  } else if constexpr (M == 2) {
    asm volatile("ds_read_b32 %0, %2 offset:0\n""ds_read_b32 %1, %2 offset:256\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]) : "v"(a) : "memory");
  } else if constexpr (M == 3) {
    asm volatile("ds_read_b32 %0, %3 offset:0\n""ds_read_b32 %1, %3 offset:256\n""ds_read_b32 %2, %3 offset:512\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]) : "v"(a) : "memory");
  } else if constexpr (M == 4) {
    asm volatile("ds_read_b32 %0, %4 offset:0\n""ds_read_b32 %1, %4 offset:256\n""ds_read_b32 %2, %4 offset:512\n""ds_read_b32 %3, %4 offset:768\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]) : "v"(a) : "memory");
  } else if constexpr (M == 5) {
    asm volatile("ds_read_b32 %0, %5 offset:0\n""ds_read_b32 %1, %5 offset:256\n""ds_read_b32 %2, %5 offset:512\n""ds_read_b32 %3, %5 offset:768\n""ds_read_b32 %4, %5 offset:1024\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]) : "v"(a) : "memory");
  } else if constexpr (M == 6) {
    asm volatile("ds_read_b32 %0, %6 offset:0\n""ds_read_b32 %1, %6 offset:256\n""ds_read_b32 %2, %6 offset:512\n""ds_read_b32 %3, %6 offset:768\n""ds_read_b32 %4, %6 offset:1024\n""ds_read_b32 %5, %6 offset:1280\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]) : "v"(a) : "memory");
  } else if constexpr (M == 7) {
    asm volatile("ds_read_b32 %0, %7 offset:0\n""ds_read_b32 %1, %7 offset:256\n""ds_read_b32 %2, %7 offset:512\n""ds_read_b32 %3, %7 offset:768\n""ds_read_b32 %4, %7 offset:1024\n""ds_read_b32 %5, %7 offset:1280\n""ds_read_b32 %6, %7 offset:1536\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]) : "v"(a) : "memory");
  } else if constexpr (M == 8) {
    asm volatile("ds_read_b32 %0, %8 offset:0\n""ds_read_b32 %1, %8 offset:256\n""ds_read_b32 %2, %8 offset:512\n""ds_read_b32 %3, %8 offset:768\n""ds_read_b32 %4, %8 offset:1024\n""ds_read_b32 %5, %8 offset:1280\n""ds_read_b32 %6, %8 offset:1536\n""ds_read_b32 %7, %8 offset:1792\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]) : "v"(a) : "memory");
  }
}
// 4 MB dwords of one row block (MFMA partials: rows 16 mb + 4 g + i, i < 4, 256 bytes apart
// per row of X, 4 KB per m block).
template <int MB>
__device__ __forceinline__ void lds_read_mb(uint32_t a, uint32_t o[4 * MB]) {
  if constexpr (MB == 1) {
    asm volatile("ds_read_b32 %0, %4 offset:0\n""ds_read_b32 %1, %4 offset:256\n""ds_read_b32 %2, %4 offset:512\n""ds_read_b32 %3, %4 offset:768\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]) : "v"(a) : "memory");
  } else if constexpr (MB == 2) {
    asm volatile("ds_read_b32 %0, %8 offset:0\n""ds_read_b32 %1, %8 offset:256\n""ds_read_b32 %2, %8 offset:512\n""ds_read_b32 %3, %8 offset:768\n""ds_read_b32 %4, %8 offset:4096\n""ds_read_b32 %5, %8 offset:4352\n""ds_read_b32 %6, %8 offset:4608\n""ds_read_b32 %7, %8 offset:4864\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]) : "v"(a) : "memory");
  } else if constexpr (MB == 3) {
    asm volatile("ds_read_b32 %0, %12 offset:0\n""ds_read_b32 %1, %12 offset:256\n""ds_read_b32 %2, %12 offset:512\n""ds_read_b32 %3, %12 offset:768\n""ds_read_b32 %4, %12 offset:4096\n""ds_read_b32 %5, %12 offset:4352\n""ds_read_b32 %6, %12 offset:4608\n""ds_read_b32 %7, %12 offset:4864\n""ds_read_b32 %8, %12 offset:8192\n""ds_read_b32 %9, %12 offset:8448\n""ds_read_b32 %10, %12 offset:8704\n""ds_read_b32 %11, %12 offset:8960\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]) : "v"(a) : "memory");
  } else if constexpr (MB == 4) {
    asm volatile("ds_read_b32 %0, %16 offset:0\n""ds_read_b32 %1, %16 offset:256\n""ds_read_b32 %2, %16 offset:512\n""ds_read_b32 %3, %16 offset:768\n""ds_read_b32 %4, %16 offset:4096\n""ds_read_b32 %5, %16 offset:4352\n""ds_read_b32 %6, %16 offset:4608\n""ds_read_b32 %7, %16 offset:4864\n""ds_read_b32 %8, %16 offset:8192\n""ds_read_b32 %9, %16 offset:8448\n""ds_read_b32 %10, %16 offset:8704\n""ds_read_b32 %11, %16 offset:8960\n""ds_read_b32 %12, %16 offset:12288\n""ds_read_b32 %13, %16 offset:12544\n""ds_read_b32 %14, %16 offset:12800\n""ds_read_b32 %15, %16 offset:13056\n" "s_waitcnt lgkmcnt(0)" : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15]) : "v"(a) : "memory");
  }
}
__device__ __forceinline__ void lds_write_u32(uint32_t a, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_write_u128(uint32_t a, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};   // a native vector: asm inputs cannot be structs
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(w) : "memory");
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

// The W reads plus the MFMA X operands of MB 16-row blocks: halves at +0 / +16 bytes, blocks
// 2 KB apart.
template <int MB>
__device__ __forceinline__ void read_stage_wmx(uint32_t ah, uint32_t al, uint32_t ax, uint4 h[4], uint2 l[4],
                                               uint4 xa[MB], uint4 xb[MB]) {
  static_assert(MB >= 1 && MB <= 4, "MFMA row blocks");
  if constexpr (MB == 1) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else if constexpr (MB == 2) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 2048) W12_X2(11, 2064) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else if constexpr (MB == 3) {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 2048) W12_X2(11, 2064) W12_X2(12, 4096)
                     W12_X2(13, 4112) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1]), "=&v"(xa[2]),
                   "=&v"(xb[2])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
  } else {
    asm volatile(W12_W_READS W12_X2(8, 0) W12_X2(9, 16) W12_X2(10, 2048) W12_X2(11, 2064) W12_X2(12, 4096)
                     W12_X2(13, 4112) W12_X2(14, 6144) W12_X2(15, 6160) "s_waitcnt lgkmcnt(0)"
                 : W12_W_OUTS(h, l), "=&v"(xa[0]), "=&v"(xb[0]), "=&v"(xa[1]), "=&v"(xb[1]), "=&v"(xa[2]),
                   "=&v"(xb[2]), "=&v"(xa[3]), "=&v"(xb[3])
                 : [ah] "v"(ah), [al] "v"(al), [ax] "v"(ax) : "memory");
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
// Step j of a segment gives lane group q (= 4 wave + lane / 16) chunk c0 + stride * j, valid
// while below c_end.  Two mappings of the segment's chunks [cs0, cs1) onto the 16 lane groups:
//  * interleaved (stride 16, c0 = cs0 + q): a wave's 4 lane groups read 4 consecutive chunks,
//    so its W bytes of a row block and X bytes of a row are contiguous;
//  * contiguous (stride 1, c0 = the start of q's share): each lane group walks its own stretch
//    of k, so its escape cursor only meets its own entries - used when the segment's escape
//    lists do not fit in LDS and are walked in global memory.
// A lane past c_end keeps reading the following chunks (inside the plane, or past it and then
// zero); that data is unused: its X is zero and its escapes are skipped.
struct SegLane {
  uint32_t c0, c_end, stride, iters;   // this lane group's chunks
  uint32_t cd0;                        // the same for lane group 4 wave + (lane >> 3) % 4 (lo DMA)
  uint32_t lo_rb0, lo_rb1;             // lo plane offsets of the row blocks this lane copies
};

// Stage j of a segment into st.  The Q pass (kQ) reads only the hi plane: the nested 8-bit
// view.
template <int RB, bool kQ>
__device__ __forceinline__ void issue_w(const GemmArgs& g, __amdgpu_buffer_rsrc_t rh, __amdgpu_buffer_rsrc_t rl,
                                        const uint32_t soff_h[RB], const SegLane& sl, uint32_t j,
                                        RingStage<RB>* st, int wave) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const uint32_t c = sl.c0 + sl.stride * j;
  const uint32_t vh = (c * kRowsPerBlock + r) * kChunkK;
  // the row block's plane offset rides in the per-lane offset: a scalar soffset would need
  // the compiler to prove it uniform, and it cannot once scalar registers run out.  The record
  // planes are read once per launch: non-temporal loads keep them from displacing X, the
  // escape slices and the partials in L2 (5-8% faster on gate_up and down, same-box A/B).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    dma16_nt(rh, &st->hi[wave][rb][0], soff_h[rb] + vh);
  if constexpr (!kQ) {
    const uint32_t cd = sl.cd0 + sl.stride * j;
    const uint32_t vl = cd * kLoChunkBytes + (lane & 7) * 16;
    dma16_nt(rl, &st->lo[wave][0], sl.lo_rb0 + vl);
    if (RB > 2) dma16_nt(rl, &st->lo[wave][64], sl.lo_rb1 + vl);
  }
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
  static constexpr int kWavesPerEU = 2;   // register budget: two work-groups per CU
  static constexpr bool kDenseOk = M <= 4;   // the escape windows' registers fit (dense instantiation)
  static constexpr bool kXInLds = true;
  static constexpr int kWStages = 2;      // W ring stages
  static constexpr int kVmemPerStage = 7;   // 6 W DMA + 1 X DMA
  typedef float Acc;
  static constexpr int kAcc = M;
  struct XStage {
    uint4 x[kWaves][kWave];   // [m][g][half]
  };
  // the lane group whose chunks this lane fetches X for (both X loads)
  __device__ static void x_groups(int wave, int lane, int& q0, int& q1) { q0 = q1 = wave * 4 + ((lane >> 1) & 3); }
  // lanes l < 8M fetch (m = l / 8, lane group l / 2 % 4, half l % 2)
  __device__ static void issue_x(const GemmArgs& g, __amdgpu_buffer_rsrc_t rx, const uint32_t xc0[2],
                                 const uint32_t xc_end[2], uint32_t stride, int /*m0*/, uint32_t j, XStage* xs,
                                 int wave) {
    const int lane = threadIdx.x & 63;
    const uint32_t m = (uint32_t)lane >> 3, half = lane & 1;
    const uint32_t c = xc0[0] + stride * j;
    const uint32_t off = (m < (uint32_t)M && c < xc_end[0]) ? (m * (uint32_t)g.ldx + c * kChunkK) * 2u + half * 16u
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
  // one stage's W bytes and X pieces of this lane
  __device__ static void read_stage(uint32_t ah, uint32_t al, const XStage* xs, int wave, uint4 h[4], uint2 l[4],
                                    uint4 xa[M], uint4 xb[M]) {
    read_stage_wx<M>(ah, al, x_addr(xs, wave), h, l, xa, xb);
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
  // red[m][row] (waves in order 0..3, called once per wave in that order).  After the
  // butterfly every lane group holds the sums of all 4 row blocks; lane group g writes row
  // block g.
  __device__ static void to_red(Acc acc[kRB][M], uint32_t red, bool first_wave) {
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    float v[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s4[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float x = acc[rb][m];
        x += __shfl_xor(x, 16, kWave);
        x += __shfl_xor(x, 32, kWave);
        s4[rb] = x;
      }
      v[m] = gq == 0 ? s4[0] : (gq == 1 ? s4[1] : (gq == 2 ? s4[2] : s4[3]));
    }
    const uint32_t a = red + (uint32_t)((gq * kRowsPerBlock + r) * 4);
    if (!first_wave) {
      uint32_t o[M];
      lds_read_m<M>(a, o);
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] += __builtin_bit_cast(float, o[m]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) lds_write_u32(a + 256u * m, __builtin_bit_cast(uint32_t, v[m]));
  }
};

// MFMA tiles: MB m blocks of 16 rows; lane (r, g) supplies X row m0 + 16 mb + r of its own
// chunk.  X rides the LDS ring like W (2 KB per wave and block), so no register load is in
// flight across a step and the compiler adds no waits of its own to the loop - except for
// two blocks, whose X is loaded one step ahead into registers (with X in LDS the LDS would
// not hold two work-groups per CU).
template <int MB>
struct MfmaPath {
  static constexpr int kMRows = MB * 16;
  static constexpr int kWavesPerEU = MB <= 2 ? 2 : 1;   // register budget: two work-groups per CU up to 32 rows
  static constexpr bool kDenseOk = MB == 1;   // the escape windows' registers fit (dense instantiation)
  // X in LDS for 16 rows (two work-groups per CU fit) and for 48-64 rows (one per CU in any
  // case: 5-7% faster than register X); 32-row tiles keep X in registers, which keeps two
  // work-groups per CU (with X in LDS they would need 98 KB each)
  static constexpr bool kXInLds = MB != 2;
  // W ring stages: three for the 64-row tiles (one work-group per CU, so LDS has room for a
  // third), keeping two W stages in flight per CU as two work-groups of the smaller tiles do
  // (measured: 4-6% faster at M = 63 / 64; no gain for the 48-row tiles, which keep two)
  static constexpr int kWStages = MB == 4 ? 3 : 2;
  static constexpr int kVmemPerStage = 6 + 2 * MB;   // 6 W DMA + 2 MB X loads
  typedef f32x4 Acc;
  static constexpr int kAcc = MB;
  struct XLds {
    uint4 x[kWaves][2 * MB * kWave];   // per wave [m block][lane group][row][half]: 32 bytes per (lane group, row)
  };
  struct XNone {};
  typedef typename std::conditional<kXInLds, XLds, XNone>::type XStage;
  // the lane groups whose chunks this lane fetches X for: load d covers lane groups 2d, 2d + 1
  __device__ static void x_groups(int wave, int lane, int& q0, int& q1) {
    q0 = wave * 4 + (lane >> 5);
    q1 = q0 + 2;
  }
  // X load (mb, d), lane l: row m0 + 16 mb + (l / 2) % 16, half l % 2 of lane group 2d + l / 32;
  // lane l of a load lands at 16 l of block mb's 2 KB, i.e. at (lane group, row, half) =
  // ((l / 32 + 2d) * 16 + row) * 32 + 16 half
  __device__ static void issue_x(const GemmArgs& g, __amdgpu_buffer_rsrc_t rx, const uint32_t xc0[2],
                                 const uint32_t xc_end[2], uint32_t stride, int m0, uint32_t j, XStage* xs,
                                 int wave) {
    if constexpr (kXInLds) {
      const int lane = threadIdx.x & 63;
      const uint32_t half = lane & 1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint32_t m = (uint32_t)(m0 + mb * 16 + ((lane >> 1) & 15));
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t c = xc0[d] + stride * j;
          const uint32_t off = (m < (uint32_t)g.M && c < xc_end[d])
                                   ? (m * (uint32_t)g.ldx + c * kChunkK) * 2u + half * 16u
                                   : kOutOfRange;
          dma16(rx, &xs->x[wave][(mb * 2 + d) * kWave], off);
        }
      }
    }
  }
  __device__ static uint32_t x_addr(const XStage* xs, int wave) {
    const int lane = threadIdx.x & 63;
    return lds_off(&xs->x[wave][0]) + (uint32_t)(((lane >> 4) * 16 + (lane & 15)) * 32);
  }
  __device__ static void read_stage(uint32_t ah, uint32_t al, const XStage* xs, int wave, uint4 h[4], uint2 l[4],
                                    uint4 xa[MB], uint4 xb[MB]) {
    if constexpr (kXInLds) read_stage_wmx<MB>(ah, al, x_addr(xs, wave), h, l, xa, xb);
    else read_stage_w(ah, al, h, l);
  }
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
  // lane (r, g) holds C[m = 16 mb + 4 g + i][n = 16 rb + r]: red[m][row] at m * 64 + row
  __device__ static void to_red(Acc acc[kRB][MB], uint32_t red, bool first_wave) {
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const uint32_t a = red + (uint32_t)((4 * gq * kTileRows + rb * kRowsPerBlock + r) * 4);
      uint32_t o[4 * MB];
      if (!first_wave) lds_read_mb<MB>(a, o);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // named components: a bit_cast of a vector-element lvalue reads element 0
        const f32x4 x = acc[rb][mb];
        float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!first_wave) v[i] += __builtin_bit_cast(float, o[4 * mb + i]);
          lds_write_u32(a + (uint32_t)(mb * 4096 + i * 256), __builtin_bit_cast(uint32_t, v[i]));
        }
      }
    }
  }
};

// ------------------------------------------------------------------------------------------
// Cross-work-group visibility without cache-wide fences: the segments of a tile may run on
// different XCDs, whose L2 caches are not coherent with each other.  Every access to the
// partial buffer and to the arrival counters is a device-scope (agent) atomic access,
// performed at the device coherence point (stores and loads carry sc1, the counter RMW is
// device-coherent), and a work-group waits for its partial stores to complete (vmcnt(0))
// before it bumps any counter.  Agent-scope release/acquire fences would write back /
// invalidate the whole L2 of the XCD instead.
// ------------------------------------------------------------------------------------------

// ------------------------------------------------------------------------------------------
// Measurement build only (-DW12_TIMELINE, libw12_timeline.so): thread 0 of every work-group
// stamps the real-time counter (100 MHz) at fixed points of the streaming kernel into slots
// of w12_timeline[work-group][16]; w12_timeline_copy reads them back.  Slots: 0 start,
// 1 prologue done, 2 / 4 first / second segment's step loop done (wave 0), 3 switch done,
// 5 / 8 the segment's last stage waited for, 6 / 9 cross-wave reduction done, 7 / 10 partial
// or Y stores issued, 11 end, 12 compute-unit id, 13 segments, 14 fixup: own stores complete,
// 15 fixup: arrival counters updated.  The normal build compiles none of this.
// ------------------------------------------------------------------------------------------
#ifdef W12_TIMELINE
__device__ unsigned long long w12_timeline[kMaxGrid * 16];
#define W12_TL(slot)                                                                           \
  do {                                                                                         \
    if (threadIdx.x == 0)                                                                      \
      w12_timeline[(size_t)blockIdx.x * 16 + (slot)] = __builtin_amdgcn_s_memrealtime();       \
  } while (0)
#define W12_TL_VAL(slot, v)                                                                    \
  do {                                                                                         \
    if (threadIdx.x == 0) w12_timeline[(size_t)blockIdx.x * 16 + (slot)] = (v);               \
  } while (0)
#else
#define W12_TL(slot) \
  do {               \
  } while (0)
#define W12_TL_VAL(slot, v) \
  do {                      \
  } while (0)
#endif

// Stream-K bookkeeping: work-group w owns units [ubeg(w), ubeg(w+1)).
__device__ __forceinline__ int64_t ubeg(const GemmArgs& g, int64_t w) { return w * g.units / g.G; }

// ------------------------------------------------------------------------------------------
// Escapes.  Each segment's 64 channels have contiguous escape lists; the slice
// [esc_ptr[row0], esc_ptr[row0 + 64]) is copied into LDS (up to kSliceEntries entries, one
// 1 KB DMA per wave) while the previous segment streams, and every lane walks a cursor over
// its channel's part of it.  A larger slice (dense escapes) is walked in global memory.
// ------------------------------------------------------------------------------------------
constexpr int kSliceEntries = kWaves * kWave * 4;   // 1024
constexpr int kMaxPend = 2;   // partial tiles of a work-group: its first and last segment

struct SegEsc {        // per lane, loaded one segment ahead
  uint2 ptr[kRB];      // {esc_ptr[n], esc_ptr[n + 1]} of the lane's 4 channels
  uint32_t base[kRB];  // window base of the lane's 4 channels
};

// The lane's channels of the segment on row group rg: esc_ptr pairs and bases, as buffer
// loads (exactly 2 kRB vector-memory instructions); rows past N read as an empty list.
__device__ __forceinline__ void load_seg_esc(const GemmArgs& g, __amdgpu_buffer_rsrc_t rp,
                                             __amdgpu_buffer_rsrc_t rbase, int64_t rg, SegEsc& se) {
  const int r = threadIdx.x & 15;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t n = rg * kTileRows + rb * kRowsPerBlock + r;
    const uint32_t po = n < g.N ? (uint32_t)n * 4u : kOutOfRange;
    se.ptr[rb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rp, (int)po, 0, 0));
    se.base[rb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rbase, (int)(n < g.N ? (uint32_t)n : kOutOfRange), 0, 0);
  }
}

// Clamp a lane's list bounds into [0, E] (rows past N: empty at E).
__device__ __forceinline__ void seg_bounds(const GemmArgs& g, int64_t rg, int rb, const SegEsc& se, uint32_t& lo,
                                           uint32_t& hi) {
  const int64_t n = rg * kTileRows + rb * kRowsPerBlock + (threadIdx.x & 15);
  if (n >= g.N) {
    lo = hi = g.num_esc;
    return;
  }
  hi = se.ptr[rb].y < g.num_esc ? se.ptr[rb].y : g.num_esc;
  lo = se.ptr[rb].x < hi ? se.ptr[rb].x : hi;
}

// First and end entry of the segment's slice (uniform): the lists of rows row0..row0+63.
__device__ __forceinline__ void slice_range(const GemmArgs& g, int64_t rg, const SegEsc& se, uint32_t& s0,
                                            uint32_t& s1) {
  uint32_t lo0, hi0, lo3, hi3;
  seg_bounds(g, rg, 0, se, lo0, hi0);
  seg_bounds(g, rg, kRB - 1, se, lo3, hi3);
  s0 = __builtin_amdgcn_readlane(lo0, 0);    // row0
  s1 = __builtin_amdgcn_readlane(hi3, 15);   // row0 + 63 (or E past N)
  s1 = s1 > s0 ? s1 : s0;
}

// One DMA per wave: entries [s0 + 256 wave, + 256) of the slice into LDS.
__device__ __forceinline__ void issue_slice(__amdgpu_buffer_rsrc_t re, uint32_t s0, uint4* slice, int wave) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)&slice[wave * kWave], 16,
                                           (int)((s0 + (uint32_t)(wave * kWave * 4 + lane * 4)) * 4u), 0, 0, 0);
}

struct LaneEsc {
  uint32_t pos, end;   // next entry and end of the channel's list (slice-relative in LDS mode)
  uint32_t e;          // the entry at pos (valid when pos < end)
};

// Cursor at the first entry with k >= k_lo.
__device__ __forceinline__ void esc_start(LaneEsc& c, const GemmArgs& g, uint32_t lo, uint32_t hi, uint32_t k_lo,
                                          bool in_lds, uint32_t s0, uint32_t slice_addr) {
  if (in_lds) {
    uint32_t pos = lo - s0, end = hi - s0;
    end = end < (uint32_t)kSliceEntries ? end : (uint32_t)kSliceEntries;   // only a malformed list exceeds it
    uint32_t e = 0;
    while (pos < end) {
      e = lds_read_u32(slice_addr + 4u * pos);
      if ((e >> 16) >= k_lo) break;
      ++pos;
    }
    c.pos = pos;
    c.end = end;
    c.e = e;
  } else {
    c.pos = lower_bound_k(g.esc, lo, hi, k_lo);
    c.end = hi;
    c.e = c.pos < c.end ? esc_global(g.esc, c.pos) : 0u;
  }
}

// Patch every escape of this lane's row that falls in chunk [k0, k0 + 16); entries below k0
// belong to other lane groups' chunks (interleaved mapping) and are stepped over.
__device__ __forceinline__ void esc_apply(LaneEsc& c, const uint32_t* __restrict__ esc, uint32_t k0, uint32_t d[8],
                                          bool in_lds, uint32_t slice_addr) {
  while (c.pos < c.end && (c.e >> 16) < k0 + kChunkK) {
    if ((c.e >> 16) >= k0) patch16(d, (c.e >> 16) - k0, c.e & 0xFFFFu);
    ++c.pos;
    if (c.pos < c.end) c.e = in_lds ? lds_read_u32(slice_addr + 4u * c.pos) : esc_global(esc, c.pos);
  }
}

// Escape-dense tensors (lists longer than the LDS slice on average) run an instantiation of
// their own, in which every segment walks its lists in global memory with the contiguous
// mapping.  Each lane keeps the next four entries of each of its lists in registers.  They
// are loaded right after a step's escapes are patched, before the next stage's loads, so the
// wait for them leaves that stage in flight (loads complete in issue order); a one-entry
// walk that waits on the spot would drain every stage in flight at each entry.  An escaped
// position holds record 0, the only record that decodes to the window base with a zero
// mantissa, so a chunk holds at most as many escapes as such values: a lane reads no more
// entries than that, and only a chunk with more than four reads past its window (one entry
// at a time, waited for on the spot).
struct EscWin {
  uint4 v;        // entries [pos, pos + 4) of the lane's list (past E: zeros, never used)
  uint32_t pos;
};

__device__ __forceinline__ void load_win(__amdgpu_buffer_rsrc_t re, const LaneEsc& c, EscWin& w) {
  w.pos = c.pos;
  const uint32_t off = c.pos < c.end ? c.pos * 4u : 0u;
  w.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(re, (int)off, 0, 0));
}

// Decoded weights of a chunk equal to the window base with a zero mantissa (record 0).
__device__ __forceinline__ uint32_t zero_records(const uint32_t d[8], uint32_t bb2) {
  uint32_t z = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t x = d[p] ^ bb2;
    z += (x & 0xFFFFu) == 0u ? 1u : 0u;
    z += (x >> 16) == 0u ? 1u : 0u;
  }
  return z;
}

// Patch the escapes of chunk [k0, k0 + 16) from the window; z bounds the entries read.
__device__ __forceinline__ void esc_apply_win(LaneEsc& c, const EscWin& w, const uint32_t* __restrict__ esc,
                                              uint32_t k0, uint32_t d[8], uint32_t z) {
  for (uint32_t i = 0; i < z; ++i) {
    if (c.pos >= c.end) break;
    const uint32_t o = c.pos - w.pos;
    const uint32_t e = o == 0u ? w.v.x : (o == 1u ? w.v.y : (o == 2u ? w.v.z : (o == 3u ? w.v.w : esc_global(esc, c.pos))));
    const uint32_t ek = e >> 16;
    if (ek >= k0 + kChunkK) break;
    if (ek >= k0) patch16(d, ek - k0, e & 0xFFFFu);
    ++c.pos;
  }
}

// Cursors of the lane's kRB lists at their first entry with k >= k_lo: the kRB binary searches
// run in lockstep, one round of loads per halving (entries through the buffer resource, so a
// finished search's probe reads nothing past E).
__device__ __forceinline__ void esc_start_lists(__amdgpu_buffer_rsrc_t re, const uint32_t lo[kRB],
                                                const uint32_t hi[kRB], uint32_t k_lo, LaneEsc c[kRB]) {
  uint32_t a[kRB], b[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    a[rb] = lo[rb];
    b[rb] = hi[rb];
    c[rb].end = hi[rb];
  }
  for (;;) {
    bool open = false;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) open = open || a[rb] < b[rb];
    if (!__builtin_amdgcn_ballot_w64(open)) break;
    uint32_t mid[kRB], v[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      mid[rb] = a[rb] + ((b[rb] - a[rb]) >> 1);
      v[rb] = __builtin_amdgcn_raw_buffer_load_b32(re, (int)(a[rb] < b[rb] ? mid[rb] * 4u : kOutOfRange), 0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (a[rb] < b[rb]) {
        if ((v[rb] >> 16) < k_lo) a[rb] = mid[rb] + 1;
        else b[rb] = mid[rb];
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) c[rb].pos = a[rb];
}

// Per-lane geometry of one segment (the stretch of one tile inside a work-group's range).
struct SegGeo {
  int64_t u, seg_end, tile, t0, rg;   // tile: index within its product; u, seg_end, t0: launch units
  int m0;
  int gi;                             // the product (group member) of the segment
  SegLane sl;
  uint32_t soff_h[kRB];
  uint32_t xc0[2], xc_end[2];   // chunks of the lane groups this lane fetches X for (Path::x_groups)
};

template <class Path>
__device__ __forceinline__ void seg_setup(const GemmArgs& g, int gi, int64_t u, int64_t u_end, bool interleaved,
                                          SegGeo& s) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int q = wave * 4 + (lane >> 4);
  s.u = u;
  s.gi = gi;
  s.tile = (u - g.ubase) / g.upt;
  s.t0 = g.ubase + s.tile * g.upt;
  s.seg_end = u_end < s.t0 + g.upt ? u_end : s.t0 + g.upt;
  s.rg = s.tile / g.MT;
  s.m0 = (int)(s.tile - s.rg * g.MT);
  // this segment's chunks [cs0, cs1) and this lane group's share of them
  const int64_t cs0 = (u - s.t0) * kUnitChunks;
  const int64_t cs1 = ((s.seg_end - s.t0) * kUnitChunks < g.Kc) ? (s.seg_end - s.t0) * kUnitChunks : g.Kc;
  SegLane& sl = s.sl;
  const int qd = wave * 4 + ((lane >> 3) & 3);
  int qx[2];
  Path::x_groups(wave, lane, qx[0], qx[1]);
  sl.c_end = (uint32_t)cs1;
  sl.iters = (uint32_t)ceil_div(cs1 - cs0, kSubRanges);
  if (interleaved) {
    sl.stride = kSubRanges;
    sl.c0 = (uint32_t)(cs0 + q);
    sl.cd0 = (uint32_t)(cs0 + qd);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      s.xc0[d] = (uint32_t)(cs0 + qx[d]);
      s.xc_end[d] = (uint32_t)cs1;
    }
  } else {
    sl.stride = 1;
    sl.c0 = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, q));
    sl.cd0 = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qd));
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      s.xc0[d] = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qx[d]));
      s.xc_end[d] = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, qx[d] + 1));
    }
    // a contiguous share ends where the next lane group's begins
    sl.c_end = (uint32_t)(cs0 + split_point(cs1 - cs0, kSubRanges, q + 1));
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    int64_t rbg = s.rg * kRB + rb;
    rbg = rbg < g.Nb ? rbg : g.Nb - 1;   // a ragged last tile re-reads its last row block
    s.soff_h[rb] = (uint32_t)(rbg * g.Kc * kHiChunkBytes);
  }
  {
    int64_t rb0 = s.rg * kRB + (lane >> 5), rb1 = s.rg * kRB + 2 + (lane >> 5);
    rb0 = rb0 < g.Nb ? rb0 : g.Nb - 1;
    rb1 = rb1 < g.Nb ? rb1 : g.Nb - 1;
    sl.lo_rb0 = (uint32_t)(rb0 * g.Kc * kLoChunkBytes);
    sl.lo_rb1 = (uint32_t)(rb1 * g.Kc * kLoChunkBytes);
  }
}

// At most `pend` vector-memory instructions may remain outstanding.  pend counts loads only
// (a stage: V, escape metadata: 2 kRB, the escape slice: 1); any other value waits for
// everything.  Leaving an instruction out of the count only makes the wait longer.
// The three-stage loop's waits: pend is a sum of (VW + VX) for the next stage's X and W, VW for
// the stage after it, 2 kRB escape-metadata loads and 1 slice DMA.
template <int VW, int VX>
__device__ __forceinline__ void wait_pending3(int pend) {
  constexpr int A = VW + VX, B = VW, E = 2 * kRB;
  if (pend == A + B) wait_vmcnt<A + B>();
  else if (pend == A + B + E) wait_vmcnt<A + B + E>();
  else if (pend == A + B + 1) wait_vmcnt<A + B + 1>();
  else if (pend == A) wait_vmcnt<A>();
  else if (pend == A + E) wait_vmcnt<A + E>();
  else if (pend == A + 1) wait_vmcnt<A + 1>();
  else if (pend == E) wait_vmcnt<E>();
  else if (pend == 1) wait_vmcnt<1>();
  else wait_vmcnt<0>();
}

// W: the escape windows' loads, issued after every stage and before its wait (dense
// instantiation), or 0.
template <int V, int W = 0>
__device__ __forceinline__ void wait_pending(int pend) {
  constexpr int E = 2 * kRB;
  if constexpr (W == 0) {
    if (pend == V + E) wait_vmcnt<V + E>();
    else if (pend == V + 1) wait_vmcnt<V + 1>();
    else if (pend == V) wait_vmcnt<V>();
    else if (pend == E) wait_vmcnt<E>();
    else if (pend == 1) wait_vmcnt<1>();
    else wait_vmcnt<0>();
  } else {
    if (pend == V + E + W) wait_vmcnt<V + E + W>();
    else if (pend == V + W) wait_vmcnt<V + W>();
    else if (pend == E + W) wait_vmcnt<E + W>();
    else if (pend == W) wait_vmcnt<W>();
    else wait_vmcnt<0>();
  }
}

// ------------------------------------------------------------------------------------------
// The kernel.
// ------------------------------------------------------------------------------------------
// kQ: the Q pass of two-level verification (news article, two-level verification part): the
// same GEMM on the nested 8-bit view, i.e. every in-window weight with its four low mantissa
// bits zero (the lo plane is never read: its ring slots hold zeros) and escapes exact.
// kDense: the instantiation for escape-dense tensors (escape windows, see EscWin).
template <class Path, bool kQ, int NG, bool kDense = false>
__device__ __forceinline__ void gemm_body(const typename ArgsOf<NG>::type& ga) {
  constexpr int RB = kRB;
  constexpr int ROWS = kTileRows;
  constexpr int MROWS = Path::kMRows;
  constexpr int V = Path::kVmemPerStage - (kQ ? 2 : 0);   // the Q pass issues no lo loads
  // loads of a stage 0 issued before a segment's epilogue (register X follows the stores)
  constexpr int V0 = Path::kXInLds ? V : V - 2 * Path::kAcc;
  constexpr int TILE_ELEMS = ROWS * MROWS;
  constexpr int ET = (TILE_ELEMS + kThreads - 1) / kThreads;   // output elements per thread
  typedef typename Path::XStage XStage;
  // Three W stages (64-row tiles): W runs two steps ahead of the stage being computed,
  // X one.  The reduction buffer then shares the second X slot, which is idle whenever red is
  // in use (a segment's end: the next segment's X stage 0 goes to the first slot), so the third
  // W stage fits in LDS.
  constexpr bool kW3 = Path::kWStages == 3;
  static_assert(!kW3 || Path::kXInLds, "three W stages need X in LDS");
  static_assert(!kDense || (Path::kDenseOk && !kW3 && NG == 1 && !kQ), "escape windows: single 2-stage products");
  constexpr int WW = kDense ? kRB : 0;   // escape-window loads between a stage and its wait
  constexpr int VW = kQ ? 4 : 6;   // W DMAs of a stage (the Q pass reads no lo plane)
  constexpr int VX = V - VW;       // X DMAs of a stage
  __shared__ RingStage<RB> ring0, ring1;
  __shared__ typename std::conditional<kW3, RingStage<RB>, char>::type ring2;
  __shared__ XStage xring0, xring1;
  __shared__ uint4 slices[2][kSliceEntries / 4];
  __shared__ float red_buf[kW3 ? 1 : TILE_ELEMS];
  static_assert(!kW3 || sizeof(XStage) >= TILE_ELEMS * sizeof(float), "red must fit the second X slot");
  __shared__ uint32_t s_flag[kMaxPend];
  __shared__ uint32_t s_pend[kMaxPend];   // tiles of this work-group's partial segments
  __shared__ uint32_t s_pendg[kMaxPend];  // and their products
  W12_TL(0);
  int tl_seg = 0;   // segments done (the timeline build's slot index)
  (void)tl_seg;
  const int wave = wave_id();
  // units, G and P are launch-wide: the same in every member of a group
  const int64_t wg = logical_wg(blockIdx.x, gridDim.x);
  const int64_t u_first = ubeg(arg_at(ga, 0), wg);
  const int64_t u_end = ubeg(arg_at(ga, 0), wg + 1);
  if (u_first >= u_end) return;
  const int gi_first = gemm_of(ga, u_first);
  // the first segment's product (the segment loop re-binds g and the resources per segment)
  const GemmArgs& g = arg_at(ga, gi_first);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(g.hi, g.hi_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(g.lo, g.lo_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.X, g.x_bytes);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(g.esc_ptr, (uint32_t)(g.N + 1) * 4u);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(g.esc, g.esc_bytes);
  const __amdgpu_buffer_rsrc_t rbase = make_rsrc(g.base, (uint32_t)g.N);
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(g.P, g.p_bytes);
  if constexpr (kQ) {
    // the lo slots of both ring stages read as zero nibbles (made visible by the prologue's
    // barrier, before any stage is read)
    uint4* lo0 = &ring0.lo[0][0];
    uint4* lo1 = &ring1.lo[0][0];
    for (int i = threadIdx.x; i < kWaves * RB * 32; i += kThreads) {
      lo0[i] = make_uint4(0, 0, 0, 0);
      lo1[i] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (kW3) {
      uint4* lo2 = &ring2.lo[0][0];
      for (int i = threadIdx.x; i < kWaves * RB * 32; i += kThreads) lo2[i] = make_uint4(0, 0, 0, 0);
    }
  }

  uint32_t ah0, al0, ah1, al1, ah2 = 0, al2 = 0;
  ring_addr<RB>(&ring0, wave, ah0, al0);
  ring_addr<RB>(&ring1, wave, ah1, al1);
  if constexpr (kW3) ring_addr<RB>(&ring2, wave, ah2, al2);
  const uint32_t slice_addr0 = lds_off(&slices[0][0]), slice_addr1 = lds_off(&slices[1][0]);
  const uint32_t red_addr = kW3 ? lds_off(&xring1) : lds_off(&red_buf[0]);

  // ---- prologue: the first segment's escape metadata and stage 0 (interleaved mapping
  // assumed), then the escape slice ----
  SegGeo cur;
  seg_setup<Path>(g, gi_first, u_first, u_end, !kDense, cur);
  uint4 xa0[Path::kAcc], xb0[Path::kAcc], xa1[Path::kAcc], xb1[Path::kAcc];
  auto issue_stage0 = [&]() {
    issue_w<RB, kQ>(g, rh, rl, cur.soff_h, cur.sl, 0, &ring0, wave);
    if constexpr (Path::kXInLds) Path::issue_x(g, rx, cur.xc0, cur.xc_end, cur.sl.stride, cur.m0 * MROWS, 0, &xring0, wave);
    else Path::load_x(g, rx, cur.m0 * MROWS, cur.sl.c0, cur.sl.c0 < cur.sl.c_end, xa0, xb0);
  };
  // the escape pointers first: the slice that depends on them completes behind stage 0 anyway
  SegEsc se;
  load_seg_esc(g, rp, rbase, cur.rg, se);
  issue_stage0();
  uint32_t s0, s1;
  slice_range(g, cur.rg, se, s0, s1);   // waits for the escape loads only (stage 0 is newer)
  if (!kDense && (s1 - s0) > (uint32_t)kSliceEntries) {
    // escape lists too long for LDS: contiguous mapping; stage 0 again (the first copy has landed)
    wait_vmcnt<0>();
    seg_setup<Path>(g, gi_first, u_first, u_end, false, cur);
    issue_stage0();
  }
  if constexpr (!kDense) issue_slice(re, s0, &slices[0][0], wave);
  if constexpr (kW3) {
    // and W stage 1, which stays in flight through the barrier
    if (cur.sl.iters > 1) {
      issue_w<RB, kQ>(g, rh, rl, cur.soff_h, cur.sl, 1, &ring1, wave);
      wait_vmcnt<VW>();
    } else {
      wait_vmcnt<0>();
    }
  } else {
    wait_vmcnt<0>();
  }
  barrier();
  W12_TL(1);

  int sb = 0;   // slice buffer of the current segment
  bool in_lds = !kDense && (s1 - s0) <= (uint32_t)kSliceEntries;
  uint32_t bb2[RB];
  LaneEsc cur_esc[RB];
  EscWin win[RB];   // dense instantiation only
  // dense instantiation: the cursors of a segment and their first windows
  auto dense_cursors = [&](const GemmArgs& gs, const SegEsc& es, __amdgpu_buffer_rsrc_t res) {
    uint32_t lo[RB], hi[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      seg_bounds(gs, cur.rg, rb, es, lo[rb], hi[rb]);
      bb2[rb] = base_pair(es.base[rb] ? es.base[rb] : 1u);
    }
    esc_start_lists(res, lo, hi, cur.sl.c0 * kChunkK, cur_esc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) load_win(res, cur_esc[rb], win[rb]);
  };
  if constexpr (kDense) {
    dense_cursors(g, se, re);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint32_t lo, hi;
      seg_bounds(g, cur.rg, rb, se, lo, hi);
      bb2[rb] = base_pair(se.base[rb] ? se.base[rb] : 1u);
      esc_start(cur_esc[rb], g, lo, hi, cur.sl.c0 * kChunkK, in_lds, s0, slice_addr0);
    }
  }
  int npend = 0;   // partial tiles listed in s_pend (the first and last segment at most)

  // The counters of the listed partial tiles go up together (one round trip); the last
  // arriver of a tile sums its partials in work-group order and writes Y.  A tile has one
  // partial slot per work-group range that meets it (that work-group's first or last segment).
  auto flush_pending = [&]() {
    wait_vm_all();   // this work-group's partial stores are complete
    __syncthreads();
    W12_TL(14);
    if (threadIdx.x < (unsigned)npend) {
      const GemmArgs& gt = arg_at(ga, NG != 1 ? s_pendg[threadIdx.x] : 0);
      const int64_t tile = s_pend[threadIdx.x];
      const int64_t t0 = gt.ubase + tile * gt.upt;
      const int64_t w_a = ceil_div((t0 + 1) * gt.G, gt.units) - 1;
      const uint32_t nsegs = (uint32_t)(ceil_div((t0 + gt.upt) * gt.G, gt.units) - w_a);
      // a split tile is the last segment of its first work-group w_a, so w_a names its counter
      const uint32_t prev = __hip_atomic_fetch_add(gt.counters + w_a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag[threadIdx.x] = (prev == nsegs - 1) ? 1u : 0u;
    }
    __syncthreads();
    W12_TL(15);
    for (int p = 0; p < npend; ++p) {
      if (!s_flag[p]) continue;
      const GemmArgs& gt = arg_at(ga, NG != 1 ? s_pendg[p] : 0);
      const int64_t tile = s_pend[p];
      const int64_t t0 = gt.ubase + tile * gt.upt;
      const int64_t w_a = ceil_div((t0 + 1) * gt.G, gt.units) - 1;
      const int64_t w_b = ceil_div((t0 + gt.upt) * gt.G, gt.units) - 1;
      const int64_t ns = w_b - w_a + 1;
      // the tile is the first segment of every contributor except possibly w_a
      const int pos_a = ubeg(gt, w_a) < t0 ? 1 : 0;
      auto slot_of = [&](int64_t j) -> int64_t { return 2 * (w_a + j) + (j == 0 ? pos_a : 0); };
      const int64_t rg = tile / gt.MT;
      const int m0 = (int)(tile - rg * gt.MT) * MROWS;
      // every load of a batch (up to 64 per thread: KB <= 16 slots x ET elements) is issued
      // before any is summed; the sum still runs in work-group order
      constexpr int KB = ET >= 64 ? 1 : (64 / ET < 16 ? 64 / ET : 16);
      float v[ET];
#pragma unroll
      for (int k = 0; k < ET; ++k) v[k] = 0.f;
      for (int64_t b0 = 0; b0 < ns; b0 += KB) {
        float pv[KB][ET];
#pragma unroll
        for (int sg = 0; sg < KB; ++sg) {
          if (b0 + sg < ns) {
            const float* src = gt.P + slot_of(b0 + sg) * (int64_t)TILE_ELEMS;
#pragma unroll
            for (int k = 0; k < ET; ++k) {
              const int e = (int)threadIdx.x + k * kThreads;
              if (e < TILE_ELEMS) pv[sg][k] = __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
#pragma unroll
        for (int sg = 0; sg < KB; ++sg) {
          if (b0 + sg < ns) {
#pragma unroll
            for (int k = 0; k < ET; ++k) v[k] = (b0 + sg == 0) ? pv[sg][k] : v[k] + pv[sg][k];
          }
        }
      }
#pragma unroll
      for (int k = 0; k < ET; ++k) {
        const int e = (int)threadIdx.x + k * kThreads;
        if (e < TILE_ELEMS) {
          const int row = e % ROWS, ml = e / ROWS;
          const int64_t n = rg * ROWS + row;
          const int m = m0 + ml;
          if (n < gt.N && m < gt.M) gt.Y[(int64_t)m * gt.ldy + n] = v[k];
        }
      }
      if (threadIdx.x == 0) __hip_atomic_store(gt.counters + w_a, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Every segment starts in ring0 / the even X registers: its stage 0 is fetched after the
  // previous segment's last step, once that step's stage is no longer read.  Its fetch follows
  // the previous segment's output stores, so no store is ever among the instructions a stage
  // wait looks past (stores and loads may complete out of order on the shared counter).
  for (;;) {
    // this segment's product and its operands (shadowing the prologue's)
    const GemmArgs& g = arg_at(ga, cur.gi);
    const Res r = make_res(g);
    const __amdgpu_buffer_rsrc_t rh = r.h, rl = r.l, rx = r.x, ry = r.y;
    // the next segment: the rest of the range, possibly in the next product
    const int64_t nu0 = cur.seg_end, nu1 = u_end;
    const bool has_next = nu0 < nu1;
    const int ngi = has_next ? gemm_from(ga, cur.gi, nu0) : cur.gi;
    const GemmArgs& ng = arg_at(ga, ngi);
    const Res nr = make_res(ng);
    const int64_t nrg = has_next ? ((nu0 - ng.ubase) / ng.upt) / ng.MT : 0;
    SegEsc nse;
    uint32_t ns0 = 0, ns1 = 0;
    typename Path::Acc acc[RB][Path::kAcc];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) Path::zero(acc[rb]);
    bool next_sliced = false;
    const uint32_t iters = cur.sl.iters;
    const uint32_t sl_addr = sb ? slice_addr1 : slice_addr0;

    // stage j is complete once at most `pend` newer vector-memory instructions remain
    // (pend < 0: the caller has waited)
    auto compute = [&](uint32_t ah, uint32_t al, const XStage* xs, uint4* xa, uint4* xb, uint32_t j, int pend) {
      if (pend >= 0) {
        if constexpr (kDense) wait_pending<V, WW>(pend + WW);
        else wait_pending<V>(pend);
      }
      static_assert(RB == 4, "ring reads are written for 4 row blocks");
      uint4 h[RB];
      uint2 l[RB];
      Path::read_stage(ah, al, xs, wave, h, l, xa, xb);
      const uint32_t c = cur.sl.c0 + cur.sl.stride * j;
      const bool valid = c < cur.sl.c_end;
      const uint32_t k0 = c * kChunkK;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t d[8];
        decode16(h[rb], l[rb], bb2[rb], d);
        if constexpr (kDense) {
          if (valid) esc_apply_win(cur_esc[rb], win[rb], g.esc, k0, d, zero_records(d, bb2[rb]));
        } else {
          if (valid) esc_apply(cur_esc[rb], g.esc, k0, d, in_lds, sl_addr);
        }
        Path::mac(d, xa, xb, acc[rb]);
      }
      if constexpr (kDense) {
        // the next step's windows, before its stage is issued
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) load_win(r.e, cur_esc[rb], win[rb]);
      }
    };
    if constexpr (kW3) {
      // stage j: W in ring j mod 3 (issued two steps ahead), X in xring j mod 2 (one step ahead)
      uint32_t wa = ah0, wl = al0, wa1 = ah1, wl1 = al1, wa2 = ah2, wl2 = al2;   // W slots of stages j, j+1, j+2
      for (uint32_t j = 0; j < iters; ++j) {
        int pend = 0;
        if (has_next && j == 0) {   // the next segment's esc_ptr pairs and bases
          load_seg_esc(ng, nr.p, nr.base, nrg, nse);
          pend += 2 * RB;
        }
        if (has_next && j == 1) {   // the next segment's escape slice (the compiler waits for the pairs)
          slice_range(ng, nrg, nse, ns0, ns1);
          issue_slice(nr.e, ns0, &slices[sb ^ 1][0], wave);
          next_sliced = true;
          pend += 1;
        }
        if (j + 1 < iters) {
          Path::issue_x(g, rx, cur.xc0, cur.xc_end, cur.sl.stride, cur.m0 * MROWS, j + 1, (j & 1) ? &xring0 : &xring1,
                        wave);
          pend += VX + VW;   // X of stage j + 1, and its W (issued a step earlier)
        }
        if (j + 2 < iters) {
          const uint32_t sw = (j + 2) % 3;
          issue_w<RB, kQ>(g, rh, rl, cur.soff_h, cur.sl, j + 2, sw == 0 ? &ring0 : (sw == 1 ? &ring1 : &ring2), wave);
          pend += VW;
        }
        // stages j complete once at most `pend` newer vector-memory instructions remain
        wait_pending3<VW, VX>(pend);
        compute(wa, wl, (j & 1) ? &xring1 : &xring0, xa0, xb0, j, -1);
        const uint32_t ta = wa, tl = wl;
        wa = wa1;
        wl = wl1;
        wa1 = wa2;
        wl1 = wl2;
        wa2 = ta;
        wl2 = tl;
      }
    } else {
    for (uint32_t j = 0; j < iters; j += 2) {
      // even step: stage j in ring0
      const bool more1 = j + 1 < iters;
      int pend = 0;
      if (more1) {
        issue_w<RB, kQ>(g, rh, rl, cur.soff_h, cur.sl, j + 1, &ring1, wave);
        if constexpr (Path::kXInLds) Path::issue_x(g, rx, cur.xc0, cur.xc_end, cur.sl.stride, cur.m0 * MROWS, j + 1, &xring1, wave);
        else {
          const uint32_t cx = cur.sl.c0 + cur.sl.stride * (j + 1);
          Path::load_x(g, rx, cur.m0 * MROWS, cx, cx < cur.sl.c_end, xa1, xb1);
        }
        pend = V;
      }
      if (has_next && j == 0) {   // the next segment's esc_ptr pairs and bases
        load_seg_esc(ng, nr.p, nr.base, nrg, nse);
        pend += 2 * RB;
      }
      compute(ah0, al0, &xring0, xa0, xb0, j, pend);
      if (!more1) break;
      // odd step: stage j + 1 in ring1
      const bool more2 = j + 2 < iters;
      pend = 0;
      if (more2) {
        issue_w<RB, kQ>(g, rh, rl, cur.soff_h, cur.sl, j + 2, &ring0, wave);
        if constexpr (Path::kXInLds) Path::issue_x(g, rx, cur.xc0, cur.xc_end, cur.sl.stride, cur.m0 * MROWS, j + 2, &xring0, wave);
        else {
          const uint32_t cx = cur.sl.c0 + cur.sl.stride * (j + 2);
          Path::load_x(g, rx, cur.m0 * MROWS, cx, cx < cur.sl.c_end, xa0, xb0);
        }
        pend = V;
      }
      if (!kDense && has_next && j == 0) {   // the next segment's escape slice (the compiler waits for the pairs)
        slice_range(ng, nrg, nse, ns0, ns1);
        issue_slice(nr.e, ns0, &slices[sb ^ 1][0], wave);
        next_sliced = true;
        pend += 1;
      }
      compute(ah1, al1, &xring1, xa1, xb1, j + 1, pend);
    }
    }

    // ---- segment end ----
    if (tl_seg < 2) W12_TL(2 + 2 * tl_seg);
    if (!kDense && has_next && !next_sliced) {   // a one-step segment
      slice_range(ng, nrg, nse, ns0, ns1);
      issue_slice(nr.e, ns0, &slices[sb ^ 1][0], wave);
    }
    // The next segment's stage 0 goes out now, so its latency overlaps the reduction and the
    // output stores below: every ring slot of this wave has been read (each stage's LDS reads
    // are waited for in the statement that issues them).  Register X (two 16-row blocks) is
    // loaded after the stores instead: the compiler waits for those registers itself, and its
    // count would include the stores.  Later stage waits count loads only, and loads complete
    // in issue order, so the stores in between can only make a wait longer.
    SegGeo nx;
    if (has_next) {
      seg_setup<Path>(ng, ngi, nu0, nu1, !kDense && (ns1 - ns0) <= (uint32_t)kSliceEntries, nx);
      issue_w<RB, kQ>(ng, nr.h, nr.l, nx.soff_h, nx.sl, 0, &ring0, wave);
      if constexpr (Path::kXInLds) Path::issue_x(ng, nr.x, nx.xc0, nx.xc_end, nx.sl.stride, nx.m0 * MROWS, 0, &xring0, wave);
      if constexpr (kW3) {
        // and its W stage 1 (the slot of red, the second X slot, is not written before the switch)
        if (nx.sl.iters > 1) {
          issue_w<RB, kQ>(ng, nr.h, nr.l, nx.soff_h, nx.sl, 1, &ring1, wave);
          wait_vmcnt<2 * VW + VX>();   // the next slice has landed (it precedes those stages)
        } else {
          wait_vmcnt<VW + VX>();
        }
      } else {
        wait_vmcnt<V0>();   // this wave's part of the next slice has landed (it precedes stage 0)
      }
    } else {
      wait_vmcnt<0>();
    }
    if (tl_seg < 2) W12_TL(5 + 3 * tl_seg);
    // red spans every wave's part of the second X slot: no wave writes it before all have read
    // their last X stage
    if constexpr (kW3) barrier();
    // waves add their partial tiles into red in wave order
    for (int w = 0; w < kWaves; ++w) {
      if (wave == w) Path::to_red(acc, red_addr, w == 0);
      wait_lgkm();
      barrier();
    }
    if (tl_seg < 2) W12_TL(6 + 3 * tl_seg);
    const bool full = (cur.u == cur.t0) && (cur.seg_end == cur.t0 + g.upt);
    const int m0 = cur.m0 * MROWS;
    // partial slot: the work-group's first or last segment
    const int64_t slot_i = 2 * wg + ((cur.u == u_first) ? 0 : 1);
    const uint32_t slot = (uint32_t)(slot_i * TILE_ELEMS);
    // buffer stores (out-of-range offsets are dropped).  red, the partial tiles and Y's rows
    // share the order e = m * 64 + row: consecutive threads touch consecutive channels.
#pragma unroll
    for (int i = 0; i < ET; ++i) {
      const int e = (int)threadIdx.x + i * kThreads;
      const bool in_tile = (TILE_ELEMS % kThreads == 0) || e < TILE_ELEMS;
      const uint32_t v = lds_read_u32(red_addr + (uint32_t)((in_tile ? e : 0) * 4));
      if (full) {
        const int row = e % ROWS, ml = e / ROWS;
        const int64_t n = cur.rg * ROWS + row;
        const int m = m0 + ml;
        const uint32_t off = (in_tile && n < g.N && m < g.M) ? (uint32_t)(((int64_t)m * g.ldy + n) * 4) : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b32(v, ry, (int)off, 0, 0);
      } else {
        // device-coherent (sc1) store: the tile's last arriver may run on another XCD
        const uint32_t off = in_tile ? (slot + (uint32_t)e) * 4u : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b32(v, rpart, (int)off, 0, kCachePolicySc1);
      }
    }
    if (!full) {
      // read after a barrier; written with explicit LDS stores, which the compiler does not
      // order behind the stage-0 DMA still in flight
      if (threadIdx.x == 0) {
        lds_write_u32(lds_off(&s_pend[0]) + 4u * (uint32_t)npend, (uint32_t)cur.tile);
        lds_write_u32(lds_off(&s_pendg[0]) + 4u * (uint32_t)npend, (uint32_t)cur.gi);
        wait_lgkm();
      }
      ++npend;
    }
    if (tl_seg < 2) W12_TL(7 + 3 * tl_seg);
    ++tl_seg;
    if (!has_next) break;
    if constexpr (!Path::kXInLds) Path::load_x(ng, nr.x, nx.m0 * MROWS, nx.sl.c0, nx.sl.c0 < nx.sl.c_end, xa0, xb0);
    wait_lgkm();
    barrier();   // red is free again; the next slice is visible to every wave
    if (tl_seg == 1) W12_TL(3);
    // switch to the next segment
    cur = nx;
    sb ^= 1;
    if constexpr (kDense) {
      dense_cursors(ng, nse, nr.e);
    } else {
      in_lds = (ns1 - ns0) <= (uint32_t)kSliceEntries;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t lo, hi;
        seg_bounds(ng, cur.rg, rb, nse, lo, hi);
        bb2[rb] = base_pair(nse.base[rb] ? nse.base[rb] : 1u);
        esc_start(cur_esc[rb], ng, lo, hi, cur.sl.c0 * kChunkK, in_lds, ns0, sb ? slice_addr1 : slice_addr0);
      }
    }
  }

  // ---- deferred split-K fixups ----
  if (npend) flush_pending();
  W12_TL(11);
  W12_TL_VAL(12, (unsigned long long)__smid());
  W12_TL_VAL(13, (unsigned long long)tl_seg);
}

template <class Path, bool kQ, bool kDense = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Path::kWavesPerEU)))
void k_gemm(GroupArgs<1> ga) {
  gemm_body<Path, kQ, 1, kDense>(ga);
}

// Up to kGroupMax independent products of the same M in one launch.
template <class Path, bool kQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Path::kWavesPerEU)))
void k_gemm_group(GroupArgs<kGroupMax> ga) {
  gemm_body<Path, kQ, kGroupMax>(ga);
}

// Any number of products, their arguments in device memory.
template <class Path, bool kQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Path::kWavesPerEU)))
void k_gemm_group_dev(GroupArgsDev ga) {
  gemm_body<Path, kQ, 0>(ga);
}

static_assert(kGroupMax == W12_GROUP_INLINE, "the kernel-argument group size is part of the C ABI");

// Stores the argument blocks of up to kGroupMax products (kernel arguments) to device memory.
__global__ __launch_bounds__(256) void k_put_args(GroupArgs<kGroupMax> c, GemmArgs* __restrict__ dst) {
  static_assert(sizeof(GemmArgs) % 4 == 0, "argument blocks are copied in 32-bit words");
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&c.g[0]);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  const int words = c.count * (int)(sizeof(GemmArgs) / 4);
  for (int i = threadIdx.x; i < words; i += blockDim.x) d[i] = src[i];
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
// Resident work-groups per CU of one kernel variant, from the runtime occupancy calculator
// (registers and LDS of the compiled kernel); when no device is visible, a conservative
// estimate.  Cached per variant.
template <class Path, bool kGroup = false>
static int occupancy_of(int fallback) {
  static std::once_flag once;
  static int v = 0;
  std::call_once(once, [fallback] {
    int n = 0;
    const void* fn = kGroup ? reinterpret_cast<const void*>(&k_gemm_group<Path, false>)
                            : reinterpret_cast<const void*>(&k_gemm<Path, false>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) == hipSuccess && n > 0)
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

template <bool kGroup>
static int groups_per_cu(int path, int M, int m_tile) {
  if (path == 1) {
    switch (M) {
      case 1: return occupancy_of<GemvPath<1>, kGroup>(2);
      case 2: return occupancy_of<GemvPath<2>, kGroup>(2);
      case 3: return occupancy_of<GemvPath<3>, kGroup>(2);
      case 4: return occupancy_of<GemvPath<4>, kGroup>(2);
      case 5: return occupancy_of<GemvPath<5>, kGroup>(2);
      case 6: return occupancy_of<GemvPath<6>, kGroup>(2);
      case 7: return occupancy_of<GemvPath<7>, kGroup>(2);
      default: return occupancy_of<GemvPath<8>, kGroup>(2);
    }
  }
  switch (m_tile / 16) {
    case 1: return occupancy_of<MfmaPath<1>, kGroup>(2);
    case 2: return occupancy_of<MfmaPath<2>, kGroup>(2);
    case 3: return occupancy_of<MfmaPath<3>, kGroup>(1);
    default: return occupancy_of<MfmaPath<4>, kGroup>(1);
  }
}

// Largest M that runs the wavefront GEMV; larger M runs MFMA tiles.  Both paths serve any
// M <= 8.  Measured on MI355X at the dense-layer shapes, the GEMV is faster for M = 1 and 2
// only: above that its per-row dot2 work grows with M while a 16-row MFMA tile costs the same
// for every M <= 16.  W12_GEMV_MAX_M (0..8) moves the boundary, e.g. 8 for the wavefront
// reduction at every M <= 8.
constexpr int kGemvMaxM = 2;

// Longest stretch of one tile (in units of 256 k) that a work-group may sum on its own: each
// lane then chains at most 16 products per unit, 4000 in all, which with the few cross-lane,
// cross-wave and split-K levels keeps every output's serial summation depth below 4096.
constexpr int64_t kMaxChainUnits = 250;

// Raise the grid so that no work-group range holds more than kMaxChainUnits units (only K
// above 64,000 needs it).
static int64_t chain_bound_grid(int64_t G, int64_t units, int64_t upt) {
  if (upt <= kMaxChainUnits) return G;
  int64_t need = ceil_div(units, kMaxChainUnits);
  need = need < kMaxGrid ? need : kMaxGrid;
  return G > need ? G : need;
}
// Smallest M that runs the wide tiles (W read once per 128 or 256 rows of X instead of once
// per 64).  W12_WIDE_MIN_M moves it.
constexpr int kWideMinM = 65;

GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K) {
  GemmPlan p{};
  int gemv_max = env_int("W12_GEMV_MAX_M", kGemvMaxM);
  gemv_max = gemv_max < 0 ? 0 : (gemv_max > 8 ? 8 : gemv_max);
  const int wide_min = env_int("W12_WIDE_MIN_M", kWideMinM);
  p.path = (M <= gemv_max) ? 1 : (M >= wide_min ? 3 : 2);
  p.rb = p.path == 3 ? kWideRB : kRB;
  p.waves = p.path == 3 ? kWideWaves : kWaves;
  const int64_t Nb = num_row_blocks(N);
  const int64_t Kc = num_chunks(K);
  p.row_groups = (Nb + p.rb - 1) / p.rb;
  if (p.path == 1) {
    p.m_tile = M;
    p.m_tiles = 1;
  } else if (p.path == 3) {
    p.m_tile = M <= 128 ? 128 : 256;
    p.m_tiles = (M + p.m_tile - 1) / p.m_tile;
  } else {
    const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 48 ? 3 : 4));
    p.m_tile = 16 * mb;
    p.m_tiles = (M + p.m_tile - 1) / p.m_tile;
  }
  p.tiles = p.row_groups * p.m_tiles;
  p.upt = (Kc + kUnitChunks - 1) / kUnitChunks;
  p.units = p.tiles * p.upt;
  const int gpc = p.path == 3 ? wide_groups_per_cu(p.m_tile) : groups_per_cu<false>(p.path, M, p.m_tile);
  int64_t G = (int64_t)device_cus() * env_int("W12_GROUPS_PER_CU", gpc);
  const int max_grid = env_int("W12_MAX_GRID", 0);   // 0: no cap
  if (max_grid > 0 && G > max_grid) G = max_grid;
  if (G > kMaxGrid) G = kMaxGrid;
  if (G > p.units) G = p.units;
  if (G < 1) G = 1;
  // When the tiles fit in the resident work-groups, use a whole multiple of them (keeping at
  // least 3/4 of the slots): every work-group then stays inside one tile, with one segment
  // and at most one partial.  A work-group whose range crosses a tile boundary pays a second
  // epilogue, a second partial and a second fixup, and the grid waits for the slowest one.
  if (p.tiles <= G) {
    const int64_t s = G / p.tiles;
    if (4 * p.tiles * s >= 3 * G) G = p.tiles * s;
  }
  G = chain_bound_grid(G, p.units, p.upt);
  p.grid = G;
  // most segments (work-group ranges) meeting one tile: 1 + the range starts strictly inside it
  {
    int64_t best = 1, run_tile = -1, run = 0;
    for (int64_t w = 1; w < G; ++w) {
      const int64_t u = w * p.units / G;
      if (u % p.upt == 0) continue;
      const int64_t t = u / p.upt;
      run = (t == run_tile) ? run + 1 : 1;
      run_tile = t;
      best = run + 1 > best ? run + 1 : best;
    }
    p.splits = (int)best;
  }
  const uint64_t tile_elems = (uint64_t)p.rb * kRowsPerBlock * (uint64_t)p.m_tile;
  p.counter_bytes = kCounterBytes;
  p.partial_bytes = 2ull * (uint64_t)G * tile_elems * sizeof(float);
  // the wide tiles: room for X in operand order (every m tile whole, zeros past M and K);
  // the other paths, ragged K: room for X padded to whole chunks
  if (p.path == 3)
    p.xpad_bytes = ((uint64_t)p.m_tiles * p.m_tile * (uint64_t)Kc * kChunkK * 2 + 255) / 256 * 256;
  else
    p.xpad_bytes = (K % kChunkK) ? ((uint64_t)M * (uint64_t)Kc * kChunkK * 2 + 255) / 256 * 256 : 0;
  p.ws_bytes = p.counter_bytes + p.partial_bytes + p.xpad_bytes;
  return p;
}

template <class Path, int NG>
static void launch_path(const GemmPlan& p, const typename ArgsOf<NG>::type& a, bool qpass, bool dense,
                        hipStream_t stream) {
  if constexpr (NG == 0) {
    if (qpass) hipLaunchKernelGGL((k_gemm_group_dev<Path, true>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_group_dev<Path, false>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
  } else if constexpr (NG == 1) {
    if constexpr (Path::kDenseOk) {
      if (dense && !qpass) {
        hipLaunchKernelGGL((k_gemm<Path, false, true>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
        return;
      }
    }
    if (qpass) hipLaunchKernelGGL((k_gemm<Path, true>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((k_gemm<Path, false>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
  } else {
    if (qpass) hipLaunchKernelGGL((k_gemm_group<Path, true>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_group<Path, false>), dim3((unsigned)p.grid), dim3(kThreads), 0, stream, a);
  }
}

template <int NG>
static void dispatch(const GemmPlan& p, int32_t M, const typename ArgsOf<NG>::type& a, bool qpass, bool dense,
                     hipStream_t stream) {
  if (p.path == 1) {
    switch (M) {
      case 1: launch_path<GemvPath<1>, NG>(p, a, qpass, dense, stream); break;
      case 2: launch_path<GemvPath<2>, NG>(p, a, qpass, dense, stream); break;
      case 3: launch_path<GemvPath<3>, NG>(p, a, qpass, dense, stream); break;
      case 4: launch_path<GemvPath<4>, NG>(p, a, qpass, dense, stream); break;
      case 5: launch_path<GemvPath<5>, NG>(p, a, qpass, dense, stream); break;
      case 6: launch_path<GemvPath<6>, NG>(p, a, qpass, dense, stream); break;
      case 7: launch_path<GemvPath<7>, NG>(p, a, qpass, dense, stream); break;
      default: launch_path<GemvPath<8>, NG>(p, a, qpass, dense, stream); break;
    }
  } else {
    switch (p.m_tile / 16) {
      case 1: launch_path<MfmaPath<1>, NG>(p, a, qpass, dense, stream); break;
      case 2: launch_path<MfmaPath<2>, NG>(p, a, qpass, dense, stream); break;
      case 3: launch_path<MfmaPath<3>, NG>(p, a, qpass, dense, stream); break;
      default: launch_path<MfmaPath<4>, NG>(p, a, qpass, dense, stream); break;
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

static void fill_args(GemmArgs& a, const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t,
                      float* Y, int64_t ldy, void* ws);

hipError_t launch_gemm(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y,
                       int64_t ldy, void* ws, bool qpass, hipStream_t stream) {
  // the wide tiles rearrange X themselves (padding included)
  if (p.path == 3) return launch_gemm_wide(p, X, M, ldx, t, Y, ldy, ws, qpass, stream);
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
  fill_args(a, p, X, M, ldx, t, Y, ldy, ws);
  a.ubase = 0;
  a.tiles = p.tiles;
  a.upt = p.upt;
  a.units = p.units;
  a.counters = reinterpret_cast<uint32_t*>(ws);
  GroupArgs<1> ga;
  ga.g[0] = a;
  ga.count = 1;
  // escape lists longer on average than the LDS slice of a 64-channel tile: the escape-window
  // instantiation (where the path has one)
  const bool dense = (uint64_t)t->num_escapes * kTileRows > (uint64_t)kSliceEntries * (uint64_t)t->N;
  dispatch<1>(p, M, ga, qpass, dense, stream);
  return hipGetLastError();
}

// The operand fields of one product (everything but its place in the launch's unit space and
// its counters).
static void fill_args(GemmArgs& a, const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t,
                      float* Y, int64_t ldy, void* ws) {
  a.Kc = num_chunks(t->K);
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
  a.G = p.grid;
  const uint64_t chunks = (uint64_t)a.Nb * (uint64_t)a.Kc;
  a.hi_bytes = (uint32_t)(chunks * kHiChunkBytes);
  a.lo_bytes = (uint32_t)(chunks * kLoChunkBytes);
  a.x_bytes = (uint32_t)(((uint64_t)(M - 1) * (uint64_t)ldx + (uint64_t)a.Kc * kChunkK) * 2u);
  a.esc_bytes = (uint32_t)((uint64_t)t->num_escapes * 4u);
  a.Y = Y;
  a.ldy = ldy;
  a.y_bytes = (uint32_t)((((uint64_t)M - 1) * (uint64_t)ldy + (uint64_t)t->N) * 4u);
  a.P = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes);
  a.p_bytes = (uint32_t)p.partial_bytes;
}

// ------------------------------------------------------------------------------------------
// Grouped launch: up to kGroupMax independent products with the same M (and K % 16 == 0,
// M <= 64: the streaming tiles) in one stream-K launch over their concatenated unit spaces.
// Launch gaps, the pipeline fill at the start and the split-K fixups at the end are paid once
// per launch instead of once per product.
// ------------------------------------------------------------------------------------------
GemmPlan plan_gemm_group(int32_t M, int32_t count, const int32_t* N, const int32_t* K, int64_t* tiles_of,
                         int64_t* upt_of) {
  GemmPlan p{};
  int gemv_max = env_int("W12_GEMV_MAX_M", kGemvMaxM);
  gemv_max = gemv_max < 0 ? 0 : (gemv_max > 8 ? 8 : gemv_max);
  p.path = M <= gemv_max ? 1 : 2;
  p.rb = kRB;
  p.waves = kWaves;
  if (p.path == 1) {
    p.m_tile = M;
    p.m_tiles = 1;
  } else {
    const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 48 ? 3 : 4));
    p.m_tile = 16 * mb;
    p.m_tiles = (M + p.m_tile - 1) / p.m_tile;
  }
  p.tiles = 0;
  p.units = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t rg = (num_row_blocks(N[i]) + p.rb - 1) / p.rb;
    tiles_of[i] = rg * p.m_tiles;
    upt_of[i] = (num_chunks(K[i]) + kUnitChunks - 1) / kUnitChunks;
    p.tiles += tiles_of[i];
    p.units += tiles_of[i] * upt_of[i];
  }
  p.row_groups = 0;
  p.upt = 0;   // per product (upt_of)
  int64_t G = (int64_t)device_cus() * env_int("W12_GROUPS_PER_CU", groups_per_cu<true>(p.path, M, p.m_tile));
  const int max_grid = env_int("W12_MAX_GRID", 0);
  if (max_grid > 0 && G > max_grid) G = max_grid;
  if (G > kMaxGrid) G = kMaxGrid;
  if (G > p.units) G = p.units;
  if (G < 1) G = 1;
  for (int i = 0; i < count; ++i) G = chain_bound_grid(G, p.units, upt_of[i]);
  p.grid = G;
  // most segments meeting one tile
  {
    int64_t best = 1, run_tile = -1, run = 0;
    int i = 0;
    int64_t ub = 0, gt = 0;   // first unit and first tile of product i (w's ranges only move forward)
    for (int64_t w = 1; w < G; ++w) {
      const int64_t uw = w * p.units / G;
      while (uw - ub >= tiles_of[i] * upt_of[i]) {
        ub += tiles_of[i] * upt_of[i];
        gt += tiles_of[i];
        ++i;
      }
      const int64_t u = uw - ub;
      if (u % upt_of[i] == 0) continue;
      const int64_t t = gt + u / upt_of[i];
      run = (t == run_tile) ? run + 1 : 1;
      run_tile = t;
      best = run + 1 > best ? run + 1 : best;
    }
    p.splits = (int)best;
  }
  const uint64_t tile_elems = (uint64_t)p.rb * kRowsPerBlock * (uint64_t)p.m_tile;
  p.counter_bytes = kCounterBytes;
  p.partial_bytes = 2ull * (uint64_t)G * tile_elems * sizeof(float);
  // more products than the kernel arguments hold: their argument blocks follow the partials
  p.xpad_bytes = count > kGroupMax ? ((uint64_t)count * sizeof(GemmArgs) + 255) / 256 * 256 : 0;
  p.ws_bytes = p.counter_bytes + p.partial_bytes + p.xpad_bytes;
  return p;
}

hipError_t launch_gemm_group(const GemmPlan& p, int32_t M, int32_t count, const w12_gemm_item* items,
                             const int64_t* tiles_of, const int64_t* upt_of, void* ws, bool qpass, hipStream_t stream) {
  if (count > kGroupMax) {
    // the arguments go to the workspace (after the partial tiles), copied on the stream
    std::vector<GemmArgs> args((size_t)count);
    int64_t ubase = 0;
    for (int i = 0; i < count; ++i) {
      GemmArgs& a = args[(size_t)i];
      fill_args(a, p, items[i].X, M, items[i].ldx, items[i].t, items[i].Y, items[i].ldy, ws);
      a.ubase = ubase;
      a.tiles = tiles_of[i];
      a.upt = upt_of[i];
      a.units = p.units;
      a.counters = reinterpret_cast<uint32_t*>(ws);
      ubase += tiles_of[i] * upt_of[i];
    }
    // stored by kernels that take them by value, kGroupMax at a time (stream-ordered, and
    // nothing on the host has to outlive the call)
    GemmArgs* dev = reinterpret_cast<GemmArgs*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes + p.partial_bytes);
    for (int c0 = 0; c0 < count; c0 += kGroupMax) {
      GroupArgs<kGroupMax> chunk{};
      chunk.count = count - c0 < kGroupMax ? count - c0 : kGroupMax;
      for (int j = 0; j < chunk.count; ++j) chunk.g[j] = args[(size_t)(c0 + j)];
      hipLaunchKernelGGL(k_put_args, dim3(1), dim3(256), 0, stream, chunk, dev + c0);
    }
    GroupArgsDev ga{dev, count};
    dispatch<0>(p, M, ga, qpass, false, stream);
    return hipGetLastError();
  }
  GroupArgs<kGroupMax> ga{};
  int64_t ubase = 0;
  for (int i = 0; i < count; ++i) {
    GemmArgs& a = ga.g[i];
    fill_args(a, p, items[i].X, M, items[i].ldx, items[i].t, items[i].Y, items[i].ldy, ws);
    a.ubase = ubase;
    a.tiles = tiles_of[i];
    a.upt = upt_of[i];
    a.units = p.units;
    a.counters = reinterpret_cast<uint32_t*>(ws);
    ubase += tiles_of[i] * upt_of[i];
  }
  for (int i = count; i < kGroupMax; ++i) ga.g[i] = ga.g[0];   // never selected (count bounds gemm_of)
  ga.count = count;
  dispatch<kGroupMax>(p, M, ga, qpass, false, stream);
  return hipGetLastError();
}

#ifdef W12_TIMELINE
hipError_t timeline_copy(void* host, uint64_t bytes) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(w12_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

}  // namespace w12
