// Device-side building blocks shared by the W12 kernels (gfx950, wave64).
//
// Format (SpecPilot summary page, method bullet of section 4.1; news article "(1) W12"):
// a weight of channel n is stored as the 12-bit record s<<11 | (e - b_n)<<7 | m when its
// exponent field e lies in the channel's 16-binade window [b_n, b_n + 15]; otherwise the
// record is 0 and the exact BF16 bits sit in the channel's escape list.
//
// Physical layout (W12_LAYOUT_RB16_K16): a 16-row x 16-k "chunk" is 256 bytes of hi
// (row-major, one byte rec >> 4 per weight) and 128 bytes of lo (8 bytes per row, the
// low nibbles arranged so that the decode below needs one byte permute per pair).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

constexpr int kRowsPerBlock = 16;   // rows of a chunk (the MFMA N dimension)
constexpr int kChunkK = 16;         // k values of a chunk held by one lane
constexpr int kHiChunkBytes = kRowsPerBlock * kChunkK;        // 256
constexpr int kLoChunkBytes = kRowsPerBlock * kChunkK / 2;    // 128
constexpr int kWave = 64;

__host__ __device__ inline int64_t num_row_blocks(int64_t n) { return (n + kRowsPerBlock - 1) / kRowsPerBlock; }
__host__ __device__ inline int64_t num_chunks(int64_t k) { return (k + kChunkK - 1) / kChunkK; }

// Byte offset of row r of chunk (row block rb, k chunk c) in the hi plane; lo is half.
__host__ __device__ inline int64_t hi_offset(int64_t rb, int64_t c, int64_t kc, int r) {
  return ((rb * kc + c) * kRowsPerBlock + r) * kChunkK;
}
__host__ __device__ inline int64_t lo_offset(int64_t rb, int64_t c, int64_t kc, int r) {
  return ((rb * kc + c) * kRowsPerBlock + r) * (kChunkK / 2);
}

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t ashr16x2(uint32_t x, short s) {
  s16x2 v = __builtin_bit_cast(s16x2, x);
  v = v >> s;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t add16x2(uint32_t x, uint32_t y) {
  u16x2 a = __builtin_bit_cast(u16x2, x), b = __builtin_bit_cast(u16x2, y);
  return __builtin_bit_cast(uint32_t, a + b);
}

// Decode 8 weights of one row of one chunk (k = 8 h .. 8 h + 7 for half h) into 4 BF16 pairs
// (natural k order: d[p] = w[2p] | w[2p+1] << 16).  hw: the half's 8 hi bytes; l: its lo word
// (lo bytes 4 h .. 4 h + 3 of the row).  bb2 = (b << 7) | (b << 23) for the channel's base b.
//
// Pair p: v_perm gathers hi bytes 2p, 2p+1 into the high byte of each 16-bit half and the
// lo bytes holding their nibbles into the low byte (nibble in bits 7..4).  An arithmetic
// shift by 4 then leaves sign in bit 15 (copied into bits 14..11), offset|mantissa in
// bits 10..0; clearing bits 14..11 and adding b << 7 gives (off + b) << 7 in the exponent
// field.  off + b <= 254, so the add never carries into the sign bit.
__device__ __forceinline__ void decode8(uint2 hw, uint32_t l, uint32_t bb2, uint32_t d[4]) {
  const uint32_t h2[2] = {hw.x, hw.y};
  const uint32_t ls = l << 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t src_lo = (p & 2) ? ls : l;
    const uint32_t sel = (p & 1) ? 0x07030602u : 0x05010400u;
    uint32_t x = __builtin_amdgcn_perm(h2[p >> 1], src_lo, sel);
    x = ashr16x2(x, 4) & 0x87FF87FFu;
    d[p] = add16x2(x, bb2);
  }
}

// The 16 weights of one row of one chunk: its two halves.
__device__ __forceinline__ void decode16(uint4 h, uint2 l, uint32_t bb2, uint32_t d[8]) {
  decode8(make_uint2(h.x, h.y), l.x, bb2, d);
  decode8(make_uint2(h.z, h.w), l.y, bb2, d + 4);
}

__device__ __forceinline__ uint32_t base_pair(uint32_t b) { return (b << 7) | (b << 23); }

// Overwrite weight `pos` (0..2W-1, may differ per lane) of W decoded BF16 pairs with `bits`.
template <int W>
__device__ __forceinline__ void patch_pairs(uint32_t d[W], uint32_t pos, uint32_t bits) {
  const uint32_t v2 = bits | (bits << 16);
  const uint32_t hm = (pos & 1u) ? 0xFFFF0000u : 0x0000FFFFu;
  const uint32_t pi = pos >> 1;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t m = (pi == (uint32_t)i) ? hm : 0u;
    d[i] = (d[i] & ~m) | (v2 & m);
  }
}
__device__ __forceinline__ void patch16(uint32_t d[8], uint32_t pos, uint32_t bits) { patch_pairs<8>(d, pos, bits); }

// First index in esc[lo, hi) whose k field is >= k0 (escapes ascend in k inside a channel).
__device__ __forceinline__ uint32_t lower_bound_k(const uint32_t* __restrict__ esc, uint32_t lo, uint32_t hi,
                                                  uint32_t k0) {
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if ((esc[mid] >> 16) < k0) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Escape range [lo, hi) of channel n, clamped so a malformed pointer array can never send
// a read outside esc[0, E).
__device__ __forceinline__ void escape_range(const uint32_t* __restrict__ esc_ptr, int64_t n, uint32_t num_esc,
                                             uint32_t& lo, uint32_t& hi) {
  uint32_t a = esc_ptr[n], b = esc_ptr[n + 1];
  hi = b < num_esc ? b : num_esc;
  lo = a < hi ? a : hi;
}

// Cursor over one channel's escape entries, walked in ascending k.
struct EscCursor {
  uint32_t idx, end;
  uint32_t next_k;     // k of the entry at idx, or 0xFFFFFFFF when exhausted
  uint32_t next_bits;
};

__device__ __forceinline__ void cursor_load(EscCursor& cur, const uint32_t* __restrict__ esc) {
  if (cur.idx < cur.end) {
    const uint32_t e = esc[cur.idx];
    cur.next_k = e >> 16;
    cur.next_bits = e & 0xFFFFu;
  } else {
    cur.next_k = 0xFFFFFFFFu;
    cur.next_bits = 0;
  }
}

// Apply every escape of the cursor with k in [k0, k0 + 16) to the decoded chunk d.  Entries
// with k < k0 are skipped (they belong to chunks this lane does not own).
__device__ __forceinline__ void cursor_apply(EscCursor& cur, const uint32_t* __restrict__ esc, uint32_t k0,
                                             uint32_t d[8]) {
  while (cur.next_k < k0 + kChunkK) {
    if (cur.next_k >= k0) patch16(d, cur.next_k - k0, cur.next_bits);
    ++cur.idx;
    cursor_load(cur, esc);
  }
}

// Load 16 BF16 values (32 bytes) starting at p; only the first `valid` are read, the rest
// are zero.  p must be 16-byte aligned when valid == 16.
__device__ __forceinline__ void load16_bf16(const uint16_t* __restrict__ p, int valid, uint4& a, uint4& b) {
  if (valid >= 16) {
    a = *reinterpret_cast<const uint4*>(p);
    b = *reinterpret_cast<const uint4*>(p + 8);
  } else {
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (2 * i < valid) ? (uint32_t)p[2 * i] : 0u;
      const uint32_t hi = (2 * i + 1 < valid) ? (uint32_t)p[2 * i + 1] : 0u;
      v[i] = lo | (hi << 16);
    }
    a = make_uint4(v[0], v[1], v[2], v[3]);
    b = make_uint4(v[4], v[5], v[6], v[7]);
  }
}

}  // namespace w12
