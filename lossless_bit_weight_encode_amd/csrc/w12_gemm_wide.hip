// W12 GEMM with wide tiles: Y[M][N] = X[M][K] . W[N][K]^T for many rows of X (batched
// verification: 128 rows and more), where the product is bound by the matrix cores rather
// than by the weight stream.
//
// Requirements from the SpecPilot summary page, method bullet of section 4.1: decode in
// registers, and a K split reduced in an order fixed in advance (identical bits run to run).
// The streaming
// kernel re-reads W once per 64 rows of X; this one reads it once per 128 or 256 rows:
//   * a work-group of 8 waves owns a tile of 64 TM rows of X (TM = 2 or 4) x 256 channels;
//     wave (wm, wn) owns rows 32 TM wm .. +32 TM and channels 64 wn .. +64, as TM x 2
//     accumulators of v_mfma_f32_32x32x16_bf16 with X as the A operand and the decoded
//     weights as the B operand;
//   * X is rearranged once per call (k_pack_x_wide) into MFMA operand order in the
//     workspace: 1 KB per 32 rows and 16 k, so that each X DMA is one contiguous 1 KB read
//     (read in place, every DMA would gather 32 separate 32-byte pieces of rows);
//   * a stage is 32 k: the X fragments of the tile and the hi/lo records of the 256 channels
//     arrive by buffer-to-LDS DMA in a ring of NS stages;
//   * each lane reads its X fragments and 8 records of each of its 2 channels from LDS,
//     decodes the records straight into the B operand and patches escapes from the segment's
//     escape slice in LDS (walked in global memory when the slice does not fit);
//   * stream-K over units of 16 chunks, as in the streaming kernel: a tile covered by several
//     work-groups gets one partial per segment, and the last to finish sums them in
//     work-group order (a fixed order set by M, N, K and the grid).
// Elements of a vector of floats are converted with __float_as_uint (by value): a bit cast of
// an element expression would read the vector's first element.
// MFMA 32x32x16 lane layout: A lane l holds row l % 32, k 8 (l / 32) .. +7; B lane l holds
// column l % 32 for the same k; D lane l holds column l % 32, rows 8 (r / 4) + 4 (l / 32) +
// r % 4 in its 16 registers r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "w12_device.h"
#include "w12_gemm_common.h"
#include "w12_kernels.h"

namespace w12 {

constexpr int kWWaves = kWideWaves;              // 8
constexpr int kWThreads = kWWaves * kWave;       // 512
constexpr int kWRB = kWideRB;                    // 16 row blocks
constexpr int kWCols = kWRB * kRowsPerBlock;     // 256 channels per tile
constexpr int kWUnitChunks = 16;                 // chunks per stream-K unit
constexpr int kWSlice = kWWaves * kWave * 4;     // escape entries held in LDS (one DMA per wave)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));

struct WideArgs {
  const uint4* X;       // X in operand order (k_pack_x_wide)
  const uint8_t* base;
  const uint8_t* hi;
  const uint8_t* lo;
  const uint32_t* esc_ptr;
  const uint32_t* esc;
  uint32_t num_esc;
  int32_t M, N, K;
  int32_t Kc, Nb;
  int32_t MT;           // m tiles
  int32_t tiles;        // row groups x m tiles
  int32_t upt;          // units per tile
  int32_t units;        // tiles x upt
  int32_t G;            // work-groups
  uint32_t hi_bytes, lo_bytes, x_bytes, esc_bytes, y_bytes, p_bytes;
  float* Y;
  int64_t ldy;
  uint32_t* counters;   // [G] arrival counters, indexed by a split tile's first work-group
  float* P;             // [2G][tile elements] partial tiles
};

// One ring stage: 32 k of the tile.
template <int TM>
struct WideStage {
  uint4 x[4 * TM][kWave];              // [kk * 2TM + mb][lane]: row 32 mb + lane % 32, k 16 kk + 8 (lane / 32)
  uint4 hi[kWRB][2][kRowsPerBlock];    // [row block][kk][row]: 16 hi bytes
  uint2 lo[kWRB][2][kRowsPerBlock];    // [row block][kk][row]: 8 lo bytes
};

template <int TM>
struct WideCfg {
  static constexpr int kRows = 64 * TM;                 // rows of X per tile
  static constexpr int kNS = TM == 4 ? 5 : 6;           // ring stages (140 / 120 KB of LDS)
  static constexpr int kXDma = TM / 2;                  // X fragments each wave fetches per stage
  static constexpr int kTile = kRows * kWCols;          // elements of a tile
  static constexpr int kF4 = 8 * TM;                    // float4 groups of accumulators per lane
};

__device__ __forceinline__ int64_t wubeg(const WideArgs& g, int64_t w) { return w * (int64_t)g.units / g.G; }

// A segment: the stretch of one tile inside a work-group's unit range.
struct WSeg {
  int64_t u, seg_end, tile, t0, rg, n0;
  int mt;             // m tile
  int mrow0;          // first row of X
  uint32_t cs0, cs1;  // chunks [cs0, cs1) of the tile's K
  uint32_t nst;       // stages (2 chunks each; the last may hold one)
};

template <int TM>
__device__ __forceinline__ void wseg(const WideArgs& g, int64_t u, int64_t u_end, WSeg& s) {
  s.u = u;
  s.tile = u / g.upt;
  s.t0 = s.tile * g.upt;
  s.seg_end = u_end < s.t0 + g.upt ? u_end : s.t0 + g.upt;
  s.rg = s.tile / g.MT;
  s.mt = (int)(s.tile - s.rg * g.MT);
  s.mrow0 = s.mt * WideCfg<TM>::kRows;
  s.n0 = s.rg * kWCols;
  s.cs0 = (uint32_t)((u - s.t0) * kWUnitChunks);
  const int64_t c1 = (s.seg_end - s.t0) * kWUnitChunks;
  s.cs1 = (uint32_t)(c1 < g.Kc ? c1 : g.Kc);
  s.nst = (s.cs1 - s.cs0 + 1) / 2;
}

// Per-lane DMA byte offsets of a segment's stage 0 (stage j adds j times 4096 TM, 512 and
// 256 bytes: two chunks of X, hi and lo); kOutOfRange for row blocks past N (the rows of X
// past M are zeros in the rearranged copy).
struct WDma {
  uint32_t x[2];     // this wave's X fragments (at most 2 per stage)
  uint32_t xkk[2];   // their chunk within the stage
  uint32_t h, l;
};

template <int TM>
__device__ __forceinline__ void wdma_setup(const WideArgs& g, const WSeg& s, int wave, int lane, WDma& d) {
#pragma unroll
  for (int i = 0; i < WideCfg<TM>::kXDma; ++i) {
    const int f = wave * WideCfg<TM>::kXDma + i;
    const int kk = f / (2 * TM), mb = f % (2 * TM);
    d.x[i] = (uint32_t)((((int64_t)s.mt * g.Kc + s.cs0 + kk) * (2 * TM) + mb) * 1024 + 16 * lane);
    d.xkk[i] = (uint32_t)kk;
  }
  const int64_t rbh = s.rg * kWRB + 2 * wave + (lane >> 5);
  d.h = rbh < g.Nb ? (uint32_t)(hi_offset(rbh, s.cs0, g.Kc, 0) + 16 * (lane & 31)) : kOutOfRange;
  const int64_t rbl = s.rg * kWRB + 4 * (wave & 3) + (lane >> 4);
  d.l = rbl < g.Nb ? (uint32_t)(lo_offset(rbl, s.cs0, g.Kc, 0) + 16 * (lane & 15)) : kOutOfRange;
}

// Stage j into st: this wave's X fragments, hi row blocks 2 wave and 2 wave + 1, and (waves
// 0-3) lo row blocks 4 wave .. 4 wave + 3.  A chunk past the segment (nch chunks) reads X as
// zero; its records are whatever follows (finite values times zero).
template <int TM, bool kQ>
__device__ __forceinline__ void wide_issue(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rh,
                                           __amdgpu_buffer_rsrc_t rl, const WDma& d, uint32_t j, uint32_t nch,
                                           WideStage<TM>* st, int wave) {
#pragma unroll
  for (int i = 0; i < WideCfg<TM>::kXDma; ++i) {
    const bool ok = d.x[i] != kOutOfRange && 2 * j + d.xkk[i] < nch;
    dma16(rx, &st->x[wave * WideCfg<TM>::kXDma + i][0], ok ? d.x[i] + (uint32_t)(4096 * TM) * j : kOutOfRange);
  }
  dma16(rh, &st->hi[2 * wave][0][0], d.h != kOutOfRange ? d.h + 512u * j : kOutOfRange);
  if (!kQ && wave < 4) dma16(rl, &st->lo[4 * wave][0][0], d.l != kOutOfRange ? d.l + 256u * j : kOutOfRange);
}

// Wait until stage j has landed for this wave: at most n newer stages (V DMAs each) remain.
template <int V, int MAXN>
__device__ __forceinline__ void wait_newer(uint32_t n) {
  if constexpr (MAXN >= 4) {
    if (n >= 4) { wait_vmcnt<4 * V>(); return; }
  }
  if constexpr (MAXN >= 3) {
    if (n == 3) { wait_vmcnt<3 * V>(); return; }
  }
  if constexpr (MAXN >= 2) {
    if (n == 2) { wait_vmcnt<2 * V>(); return; }
  }
  if (n == 1) { wait_vmcnt<V>(); return; }
  wait_vmcnt<0>();
}

// One k16 step of a wave: its TM X fragments (1 KB apart) and, for its 2 channel blocks, 8 hi
// bytes (blocks 1 KB apart) and 4 lo bytes (512 bytes apart), in one statement with its wait.
#define W12W_A(i, off) "ds_read_b128 %" #i ", %[ax] offset:" #off "\n"
#define W12W_B(ih, il)                                                                       \
  "ds_read_b64 %" #ih ", %[ah] offset:0\n"                                                   \
  "ds_read_b64 %" #il ", %[ah] offset:1024\n"
#define W12W_L(i0, i1)                                                                       \
  "ds_read_b32 %" #i0 ", %[al] offset:0\n"                                                   \
  "ds_read_b32 %" #i1 ", %[al] offset:512\n"
template <int TM, bool kQ>
__device__ __forceinline__ void read_step(uint32_t ax, uint32_t ah, uint32_t al, uint4 a[TM], uint2 h[2],
                                          uint32_t l[2]) {
  static_assert(TM == 2 || TM == 4, "tile rows");
  if constexpr (kQ) {
    l[0] = l[1] = 0u;
    if constexpr (TM == 2) {
      asm volatile(W12W_A(0, 0) W12W_A(1, 1024) W12W_B(2, 3) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(a[0]), "=&v"(a[1]), "=&v"(h[0]), "=&v"(h[1])
                   : [ax] "v"(ax), [ah] "v"(ah) : "memory");
    } else {
      asm volatile(W12W_A(0, 0) W12W_A(1, 1024) W12W_A(2, 2048) W12W_A(3, 3072) W12W_B(4, 5) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(h[0]), "=&v"(h[1])
                   : [ax] "v"(ax), [ah] "v"(ah) : "memory");
    }
  } else {
    if constexpr (TM == 2) {
      asm volatile(W12W_A(0, 0) W12W_A(1, 1024) W12W_B(2, 3) W12W_L(4, 5) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(a[0]), "=&v"(a[1]), "=&v"(h[0]), "=&v"(h[1]), "=&v"(l[0]), "=&v"(l[1])
                   : [ax] "v"(ax), [ah] "v"(ah), [al] "v"(al) : "memory");
    } else {
      asm volatile(W12W_A(0, 0) W12W_A(1, 1024) W12W_A(2, 2048) W12W_A(3, 3072) W12W_B(4, 5) W12W_L(6, 7)
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(h[0]), "=&v"(h[1]), "=&v"(l[0]),
                     "=&v"(l[1])
                   : [ax] "v"(ax), [ah] "v"(ah), [al] "v"(al) : "memory");
    }
  }
}
#undef W12W_A
#undef W12W_B
#undef W12W_L

// Escape cursor of one lane over one channel's list (slice-relative positions in LDS mode).
struct WEsc {
  uint32_t pos, end, e;   // e: the entry at pos (valid when pos < end)
  uint32_t nk;            // k of the entry at pos, all ones once the list is done
};

__device__ __forceinline__ void wesc_start(WEsc& c, const uint32_t* __restrict__ esc, uint32_t lo, uint32_t hi,
                                           uint32_t k_lo, bool in_lds, uint32_t s0, uint32_t slice_addr) {
  if (in_lds) {
    uint32_t pos = lo - s0, end = hi - s0;
    end = end < (uint32_t)kWSlice ? end : (uint32_t)kWSlice;   // only a malformed list exceeds it
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
    c.pos = lower_bound_k(esc, lo, hi, k_lo);
    c.end = hi;
    c.e = c.pos < c.end ? esc_global(esc, c.pos) : 0u;
  }
  c.nk = c.pos < c.end ? c.e >> 16 : 0xFFFFFFFFu;
}

// Consume the entries of chunk [k16, k16 + 16); patch those in this lane's half
// [k16 + 8 h, + 8) into its 4 decoded pairs.
__device__ __forceinline__ void wesc_apply(WEsc& c, const uint32_t* __restrict__ esc, uint32_t k16, uint32_t kh,
                                           uint32_t d[4], bool in_lds, uint32_t slice_addr) {
  while (c.nk < k16 + kChunkK) {
    const uint32_t k = c.nk;
    if (k >= kh && k < kh + 8) patch_pairs<4>(d, k - kh, c.e & 0xFFFFu);
    ++c.pos;
    if (c.pos < c.end) {
      c.e = in_lds ? lds_read_u32(slice_addr + 4u * c.pos) : esc_global(esc, c.pos);
      c.nk = c.e >> 16;
    } else {
      c.nk = 0xFFFFFFFFu;
    }
  }
}

// Escape-dense tensors (lists longer than the LDS slice on average) run an instantiation of
// their own.  There every list is walked in global memory, and a cursor's next entry read on the
// spot waits for every load in flight (loads complete in issue order), which would drain the
// ring at nearly every step.  Instead each stage's DMAs also gather, for each of the tile's 256
// channels, the kWWin entries from the channel's cursor as it stands when the stage is issued
// (the wave of row half wm takes the channels of block nb = wm, 16 bytes per lane); the entries
// a stage needs are then in its window unless the channel holds more than kWWin entries in the
// stages in flight, and only those are read from global memory.
constexpr int kWWin = 8;   // entries per channel gathered with each stage (two 16-byte halves)

__device__ __forceinline__ void lds_write_u32_w(uint32_t a, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1\ns_waitcnt lgkmcnt(0)" : : "v"(a), "v"(v) : "memory");
}

// wesc_apply with the next entries from the stage's window: win is the channel's window
// (entries 0-3 at win, 4-7 at win + 512), wp the list position of its first entry.
__device__ __forceinline__ void wesc_apply_win(WEsc& c, const uint32_t* __restrict__ esc, uint32_t k16, uint32_t kh,
                                               uint32_t d[4], uint32_t win, uint32_t wp) {
  while (c.nk < k16 + kChunkK) {
    const uint32_t k = c.nk;
    if (k >= kh && k < kh + 8) patch_pairs<4>(d, k - kh, c.e & 0xFFFFu);
    ++c.pos;
    if (c.pos < c.end) {
      const uint32_t o = c.pos - wp;   // the cursor never moves back past the window's start
      c.e = o < (uint32_t)kWWin ? lds_read_u32(win + (o >= 4u ? 512u : 0u) + 4u * (o & 3u)) : esc_global(esc, c.pos);
      c.nk = c.e >> 16;
    } else {
      c.nk = 0xFFFFFFFFu;
    }
  }
}

// Output element (i, nb, r) of this lane: row and channel inside the tile.
template <int TM>
__device__ __forceinline__ int out_row(int wm, int i, int r, int lane) {
  return 32 * (wm * TM + i) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int out_col(int wn, int nb, int lane) { return 64 * wn + 32 * nb + (lane & 31); }

// kQ: the Q pass on the nested 8-bit view (lo plane never read: zero nibbles; escapes exact).
// kDense: the instantiation for escape-dense tensors (escape windows gathered with each stage,
// a ring of 4 stages to make room for them).
template <int TM, bool kQ, bool kDense = false>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_wide(WideArgs g) {
  typedef WideCfg<TM> C;
  static_assert(!(kDense && kQ), "escape windows: exact pass only");
  constexpr int NS = kDense ? 4 : C::kNS;
  constexpr int VW = kDense ? 1 : 0;                       // the window DMA of a stage
  constexpr int V_LO = C::kXDma + 1 + (kQ ? 0 : 1) + VW;   // DMAs per stage of waves 0-3
  constexpr int V_NL = C::kXDma + 1 + VW;                  // of waves 4-7
  __shared__ WideStage<TM> ring[NS];
  __shared__ uint32_t slice[kDense ? 4 : kWSlice];
  __shared__ uint4 wwin[kDense ? NS : 1][kWCols / 32][kWave];   // [stage][block of 32 channels][half, channel]
  __shared__ uint32_t wwpos[kDense ? NS : 1][kWCols];          // [stage][channel]: list position of the window
  __shared__ uint32_t s_last;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const uint32_t hsel = (uint32_t)(lane >> 5);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(g.hi, g.hi_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(g.lo, g.lo_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.X, g.x_bytes);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(g.esc, g.esc_bytes);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(g.Y, g.y_bytes);
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(g.P, g.p_bytes);

  const int64_t u_first = wubeg(g, blockIdx.x);
  const int64_t u_end = wubeg(g, (int64_t)blockIdx.x + 1);
  if (u_first >= u_end) return;
  const uint32_t slice_addr = lds_off(&slice[0]);
  // this lane's LDS read addresses in ring stage 0 (k16 step 0); stage s adds s * sizeof
  const uint32_t ax0 = lds_off(&ring[0].x[wm * TM][lane]);
  const int rb_l = 4 * wn + ((lane & 31) >> 4), row_l = lane & 15;
  const uint32_t ah0 = lds_off(&ring[0].hi[rb_l][0][row_l]) + 8u * hsel;
  const uint32_t al0 = lds_off(&ring[0].lo[rb_l][0][row_l]) + 4u * hsel;
  constexpr uint32_t kStageBytes = sizeof(WideStage<TM>);

  int64_t u = u_first;
  for (;;) {
    WSeg s;
    wseg<TM>(g, u, u_end, s);

    // ---- escape metadata: the slice of the tile's 256 channels, the lane's 2 channels ----
    const int64_t n_hi = s.n0 + kWCols < g.N ? s.n0 + kWCols : g.N;
    uint32_t s1 = __builtin_amdgcn_readfirstlane(g.esc_ptr[n_hi]);
    uint32_t s0 = __builtin_amdgcn_readfirstlane(g.esc_ptr[s.n0]);
    s1 = s1 < g.num_esc ? s1 : g.num_esc;
    s0 = s0 < s1 ? s0 : s1;
    const bool in_lds = !kDense && (s1 - s0) <= (uint32_t)kWSlice;
    uint32_t elo[2], ehi[2], bb2[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t n = s.n0 + out_col(wn, nb, lane);
      if (n < g.N) {
        escape_range(g.esc_ptr, n, g.num_esc, elo[nb], ehi[nb]);
        const uint32_t b = g.base[n];
        bb2[nb] = base_pair(b ? b : 1u);
      } else {
        elo[nb] = ehi[nb] = g.num_esc;
        bb2[nb] = base_pair(1u);
      }
    }
    if (in_lds) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)&slice[wave * kWave * 4], 16,
                                               (int)((s0 + (uint32_t)(wave * kWave * 4 + lane * 4)) * 4u), 0, 0, 0);
    }
    WEsc cur[2];
    if constexpr (kDense) {   // global-memory cursors, before the stages (their windows start there)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) wesc_start(cur[nb], g.esc, elo[nb], ehi[nb], s.cs0 * kChunkK, false, s0, slice_addr);
    }
    // the window of a stage: this wave's channel block nb = wm, from each cursor as it stands
    auto issue_win = [&](uint32_t slot_w) {
      if constexpr (kDense) {
        const uint32_t pos = wm ? cur[1].pos : cur[0].pos;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)&wwin[slot_w][2 * wn + wm][0], 16,
                                                 (int)((pos + 4u * hsel) * 4u), 0, 0, 0);
        if (lane < 32) lds_write_u32_w(lds_off(&wwpos[slot_w][64 * wn + 32 * wm + lane]), pos);
      }
    };
    // ---- the first NS - 1 stages ----
    WDma dm;
    wdma_setup<TM>(g, s, wave, lane, dm);
    const uint32_t nch = s.cs1 - s.cs0;
    for (uint32_t j = 0; j < (uint32_t)(NS - 1) && j < s.nst; ++j) {
      wide_issue<TM, kQ>(rx, rh, rl, dm, j, nch, &ring[j], wave);
      issue_win(j);
    }
    wait_vm_all();
    barrier();
    if constexpr (!kDense) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) wesc_start(cur[nb], g.esc, elo[nb], ehi[nb], s.cs0 * kChunkK, in_lds, s0, slice_addr);
    }

    f32x16 acc[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][nb][r] = 0.f;

    uint32_t slot = 0;   // ring slot of stage j
    for (uint32_t j = 0; j < s.nst; ++j) {
      // stage j has landed once at most min(NS - 2, stages after it) newer stages remain
      const uint32_t left = s.nst - 1 - j;
      const uint32_t newer = left < (uint32_t)(NS - 2) ? left : (uint32_t)(NS - 2);
      if (wave < 4) wait_newer<V_LO, NS - 2>(newer);
      else wait_newer<V_NL, NS - 2>(newer);
      barrier();   // stage j visible to all waves; every wave is done with stage j - 1
      if (j + NS - 1 < s.nst) {
        const uint32_t ws = slot == 0 ? NS - 1 : slot - 1;
        wide_issue<TM, kQ>(rx, rh, rl, dm, j + NS - 1, nch, &ring[ws], wave);
        issue_win(ws);
      }
      // one test per stage: does any lane of the wave hold an escape before the stage's end?
      // (each cursor carries the k of its next entry; then one test per k16 step and channel
      // block, so only the lists that have an entry there are walked)
      const uint32_t kend = (s.cs0 + 2 * j + 2) * kChunkK;
      const bool any_esc = __builtin_amdgcn_ballot_w64(min(cur[0].nk, cur[1].nk) < kend) != 0;
      const uint32_t so = slot * kStageBytes;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint4 a[TM];
        uint2 h[2];
        uint32_t l[2];
        read_step<TM, kQ>(ax0 + so + kk * (2 * TM * kWave * 16), ah0 + so + kk * 256, al0 + so + kk * 128, a, h, l);
        uint32_t d[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) decode8(h[nb], l[nb], bb2[nb], d[nb]);
        const uint32_t ck = s.cs0 + 2 * j + kk;
        if (any_esc && ck < s.cs1) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            if (__builtin_amdgcn_ballot_w64(cur[nb].nk < (ck + 1) * kChunkK) != 0) {
              if constexpr (kDense) {
                const uint32_t cw = 64 * wn + 32 * nb + (lane & 31);
                wesc_apply_win(cur[nb], g.esc, ck * kChunkK, ck * kChunkK + 8 * hsel, d[nb],
                               lds_off(&wwin[slot][2 * wn + nb][lane & 31]), lds_read_u32(lds_off(&wwpos[slot][cw])));
              } else {
                wesc_apply(cur[nb], g.esc, ck * kChunkK, ck * kChunkK + 8 * hsel, d[nb], in_lds, slice_addr);
              }
            }
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(d[nb][0], d[nb][1], d[nb][2], d[nb][3]));
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[i][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]), b, acc[i][nb], 0, 0, 0);
        }
      }
      slot = slot == NS - 1 ? 0 : slot + 1;
    }

    // ---- segment end ----
    const bool full = (s.u == s.t0) && (s.seg_end == s.t0 + g.upt);
    if (full) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = s.mrow0 + out_row<TM>(wm, i, r, lane);
            const int64_t n = s.n0 + out_col(wn, nb, lane);
            const uint32_t off = (m < g.M && n < g.N) ? (uint32_t)(((int64_t)m * g.ldy + n) * 4) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][nb][r]), ry, (int)off, 0, 0);
          }
    } else {
      // partial slot: the work-group's first or last segment; layout [float4 group][thread]
      const int64_t slot_i = 2 * (int64_t)blockIdx.x + ((s.u == u_first) ? 0 : 1);
      const uint32_t pbase = (uint32_t)(slot_i * C::kTile);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int grp = (i * 2 + nb) * 4 + q;
            const uint32_t off = (pbase + (uint32_t)(grp * kWThreads + (int)threadIdx.x) * 4u) * 4u;
            const uint4 v = make_uint4(__float_as_uint(acc[i][nb][4 * q]),
                                       __float_as_uint(acc[i][nb][4 * q + 1]),
                                       __float_as_uint(acc[i][nb][4 * q + 2]),
                                       __float_as_uint(acc[i][nb][4 * q + 3]));
            // device-coherent (sc1) store: the tile's last arriver may run on another XCD
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4w, v), rpart, (int)off, 0, kCachePolicySc1);
          }
      wait_vm_all();   // this work-group's partial stores are complete
      __syncthreads();
      const int64_t t0 = s.t0;
      const int64_t w_a = ceil_div((t0 + 1) * g.G, g.units) - 1;
      const int64_t w_b = ceil_div((t0 + g.upt) * g.G, g.units) - 1;
      const int64_t ns = w_b - w_a + 1;
      if (threadIdx.x == 0) {
        // the tile's counter is its first work-group's (the tile is w_a's last segment)
        const uint32_t prev = __hip_atomic_fetch_add(g.counters + w_a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(ns - 1)) ? 1u : 0u;
      }
      __syncthreads();
      if (s_last) {
        // the last arriver: sum the tile's partials in work-group order and write Y.  Per
        // contributor, the loads of 8 of this thread's float4 groups are in flight at once.
        const int pos_a = wubeg(g, w_a) < t0 ? 1 : 0;
        constexpr int HG = 8;   // float4 groups per batch
#pragma unroll
        for (int half = 0; half < C::kF4 / HG; ++half) {
          f32x4 v[HG];
          for (int64_t jj = 0; jj < ns; ++jj) {
            const int64_t sl = 2 * (w_a + jj) + (jj == 0 ? pos_a : 0);
            const uint32_t sbase = (uint32_t)(sl * C::kTile);
            f32x4 pv[HG];
#pragma unroll
            for (int x = 0; x < HG; ++x) {
              const int grp = half * HG + x;
              const uint32_t off = (sbase + (uint32_t)(grp * kWThreads + (int)threadIdx.x) * 4u) * 4u;
              pv[x] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rpart, (int)off, 0, kCachePolicySc1));
            }
#pragma unroll
            for (int x = 0; x < HG; ++x) v[x] = (jj == 0) ? pv[x] : v[x] + pv[x];
          }
#pragma unroll
          for (int x = 0; x < HG; ++x) {
            const int grp = half * HG + x;
            const int i = grp / 8, nb = (grp / 4) % 2, q = grp % 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = s.mrow0 + out_row<TM>(wm, i, 4 * q + e, lane);
              const int64_t n = s.n0 + out_col(wn, nb, lane);
              const uint32_t off = (m < g.M && n < g.N) ? (uint32_t)(((int64_t)m * g.ldy + n) * 4) : kOutOfRange;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[x][e]), ry, (int)off, 0, 0);
            }
          }
        }
        if (threadIdx.x == 0) __hip_atomic_store(g.counters + w_a, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    u = s.seg_end;
    if (u >= u_end) break;
    barrier();   // every wave is done with the ring and the slice before the next segment's DMAs
  }
}

// X rearranged for the wide tiles.  Fragment (t, c, b), 1 KB at ((t Kc + c) 2TM + b) KB,
// holds for lane l the 8 elements of row 64 TM t + 32 b + l % 32 at k = 16 c + 8 (l / 32)
// .. + 7, zeros past M and K: what lane l of the A operand of v_mfma_f32_32x32x16_bf16 takes
// for rows 32 b .. + 31 and k 16 c .. + 15 of m tile t.  One thread per 8 elements of a row,
// in row order (coalesced reads, 16-byte writes).
template <int TM>
__global__ __launch_bounds__(256) void k_pack_x_wide(const uint16_t* __restrict__ X, int64_t ldx, int32_t M,
                                                     int32_t K, int32_t Kc, int64_t rows, uint4* __restrict__ out) {
  const int64_t groups = 2 * (int64_t)Kc;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * groups) return;
  const int64_t m = i / groups;
  const int g = (int)(i - m * groups);
  const int64_t k0 = 8 * (int64_t)g;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (m < M) {
    const uint16_t* p = X + m * ldx + k0;
    if (k0 + 8 <= K && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
      v = *reinterpret_cast<const uint4*>(p);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = k0 + 2 * j < K ? p[2 * j] : 0u;
        const uint32_t b = k0 + 2 * j + 1 < K ? p[2 * j + 1] : 0u;
        w[j] = a | (b << 16);
      }
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  const int64_t t = m / WideCfg<TM>::kRows;
  const int r = (int)(m - t * WideCfg<TM>::kRows);
  const int lane = (r & 31) + 32 * (g & 1);
  out[((t * Kc + (g >> 1)) * (2 * TM) + (r >> 5)) * kWave + lane] = v;
}

template <int TM, bool kQ = false>
static int occupancy_wide(int fallback) {
  static std::once_flag once;
  static int v = 0;
  std::call_once(once, [fallback] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&k_gemm_wide<TM, kQ>),
                                                     kWThreads, 0) == hipSuccess &&
        n > 0)
      v = n;
    else {
      (void)hipGetLastError();
      v = fallback;
    }
  });
  return v;
}

int wide_groups_per_cu(int m_tile) { return m_tile <= 128 ? occupancy_wide<2>(1) : occupancy_wide<4>(1); }

hipError_t launch_gemm_wide(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t,
                            float* Y, int64_t ldy, void* ws, bool qpass, hipStream_t stream) {
  WideArgs a;
  a.Kc = (int32_t)num_chunks(t->K);
  // X into operand order, in the workspace after the partials
  uint4* xp = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes + p.partial_bytes);
  const int64_t rows = (int64_t)p.m_tiles * p.m_tile;
  const int64_t threads = rows * 2 * a.Kc;
  const dim3 pgrid((unsigned)((threads + 255) / 256)), pblock(256);
  if (p.m_tile <= 128) hipLaunchKernelGGL((k_pack_x_wide<2>), pgrid, pblock, 0, stream, X, ldx, M, t->K, a.Kc, rows, xp);
  else hipLaunchKernelGGL((k_pack_x_wide<4>), pgrid, pblock, 0, stream, X, ldx, M, t->K, a.Kc, rows, xp);
  a.X = xp;
  a.base = t->base;
  a.hi = t->hi;
  a.lo = t->lo;
  a.esc_ptr = t->esc_ptr;
  a.esc = t->esc;
  a.num_esc = (uint32_t)t->num_escapes;
  a.M = M;
  a.N = t->N;
  a.K = t->K;
  a.Nb = (int32_t)num_row_blocks(t->N);
  a.MT = p.m_tiles;
  a.tiles = (int32_t)p.tiles;
  a.upt = (int32_t)p.upt;
  a.units = (int32_t)p.units;
  a.G = (int32_t)p.grid;
  const uint64_t chunks = (uint64_t)a.Nb * (uint64_t)a.Kc;
  a.hi_bytes = (uint32_t)(chunks * kHiChunkBytes);
  a.lo_bytes = (uint32_t)(chunks * kLoChunkBytes);
  a.x_bytes = (uint32_t)((uint64_t)rows * (uint64_t)a.Kc * kChunkK * 2u);
  a.esc_bytes = (uint32_t)((uint64_t)t->num_escapes * 4u);
  a.Y = Y;
  a.ldy = ldy;
  a.y_bytes = (uint32_t)((((uint64_t)M - 1) * (uint64_t)ldy + (uint64_t)t->N) * 4u);
  a.counters = reinterpret_cast<uint32_t*>(ws);
  a.P = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes);
  a.p_bytes = (uint32_t)p.partial_bytes;
  const dim3 grid((unsigned)p.grid), block(kWThreads);
  // escape lists longer on average than the LDS slice of a 256-channel tile: the escape-window
  // instantiation (exact pass)
  const bool dense = !qpass && (uint64_t)t->num_escapes * kWCols > (uint64_t)kWSlice * (uint64_t)t->N;
  if (p.m_tile <= 128) {
    if (qpass) hipLaunchKernelGGL((k_gemm_wide<2, true>), grid, block, 0, stream, a);
    else if (dense) hipLaunchKernelGGL((k_gemm_wide<2, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_wide<2, false>), grid, block, 0, stream, a);
  } else {
    if (qpass) hipLaunchKernelGGL((k_gemm_wide<4, true>), grid, block, 0, stream, a);
    else if (dense) hipLaunchKernelGGL((k_gemm_wide<4, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_wide<4, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace w12
