// W12 encode kernels: per-channel window choice, escape-count scan, record emission.
//
// The record (SpecPilot summary page, method bullet of section 4.1) keeps a weight's sign, its
// exponent as a 4-bit offset from the channel's window base (a window of 16 binades) and the
// top 7 mantissa bits; the weights a record cannot hold (exponent outside the window, zero,
// subnormal) go to an exact side list.  Per the news article, part "(1) W12", the exponents of
// one output channel sit close together, which is what makes a per-channel window pay.  The
// window base b of a channel is the smallest b in 1..239 that maximises the number of weights
// with exponent field in [b, b+15].
#include "w12_device.h"
#include "w12_gemm_common.h"
#include "w12_kernels.h"

namespace w12 {

// Two BF16 weights share a 32-bit word (the lower k in the low half); both are handled at once
// with packed 16-bit integer arithmetic, which never carries between the halves.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t bits_of(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t bits_of(i16x2 x) { return __builtin_bit_cast(uint32_t, x); }

constexpr int kCountWaves = 4;
constexpr int kCountBatch = 8;    // 16-byte loads per lane in flight before they are counted
constexpr int kBandBins = 16;     // exponent fields counted in lane-private counters
constexpr int kBandBelow = 12;    // the band starts this many fields below the lanes' median maximum
constexpr int kBandStride = kCountWaves * kWave;   // words between a thread's band counters

// A field e outside the band [lo, lo + 15] was added to band counter e & 15 like the others:
// take it back there and count it in the wave's shared histogram instead (fields 0 and 255 are
// in no window and are dropped).
__device__ __forceinline__ void count_outside(uint32_t e, uint32_t lo, uint32_t* __restrict__ band,
                                              uint32_t* __restrict__ hist) {
  if (e - lo >= (uint32_t)kBandBins) {
    atomicSub(band + (e & (kBandBins - 1)) * kBandStride, 1u);
    if (e != 0u && e != 255u) atomicAdd(hist + e, 1u);
  }
}

// One wave per channel: exponent counts, then the best 16-wide window.  A channel's exponents
// sit in a handful of fields, so 64 lanes adding to one shared histogram would mostly hit the
// same few words.  Instead each lane adds every field e to a counter of its own, number e & 15,
// which is exact for the fields of a 16-field band [lo, lo + 15] (they map one to one onto the
// 16 counters); the counters are laid out [counter][thread], so no other lane shares them and a
// wave's additions fall in distinct banks.  A packed test, two fields at a time, flags the rare
// fields outside the band; once per 8 weights of a lane, if any lane of the wave has one, they
// are moved to the shared histogram.  The band is placed from the first load: its base lies
// kBandBelow fields below the median over the lanes of each lane's largest field, so it covers
// the channel's bulk even when a few large outliers are present.  A field outside the band is
// still counted exactly, only more slowly.  Each lane issues kCountBatch loads (8 KB per wave)
// before counting them.  They keep the default cache policy: what they leave in the caches
// serves the emit, which reads W next.  At the end the lanes' counters are summed into the
// histogram, and the window counts of all bases come from one prefix sum over the 256 fields.
__global__ __launch_bounds__(kCountWaves * kWave) void k_encode_count(
    const uint16_t* __restrict__ W, int32_t N, int32_t K, int64_t ldw, const uint8_t* __restrict__ forced,
    uint8_t* __restrict__ base, uint32_t* __restrict__ esc_ptr) {
  __shared__ uint32_t s_band[kBandBins][kBandStride];   // [counter][thread]
  __shared__ __align__(16) uint32_t s_hist[kCountWaves][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * kCountWaves + wave;
  if (n >= N) return;   // no work-group barrier follows: every wave works on LDS of its own
  uint32_t* const band = &s_band[0][threadIdx.x];
  uint32_t* const hist = s_hist[wave];
#pragma unroll
  for (int i = 0; i < kBandBins; ++i) band[i * kBandStride] = 0;
  reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0, 0, 0, 0);
  const uint16_t* row = W + n * ldw;
  const int full = K / 8;   // whole 8-element groups
  uint32_t lo = 0;
  for (int g0 = 0; g0 < full; g0 += kCountBatch * kWave) {
    uint4 q[kCountBatch];
#pragma unroll
    for (int i = 0; i < kCountBatch; ++i) {
      const int gi = g0 + i * kWave + lane;
      q[i] = gi < full ? *reinterpret_cast<const uint4*>(row + 8 * gi) : make_uint4(0, 0, 0, 0);
    }
    if (g0 == 0) {
      // the band: the median over the lanes with data of their largest field below 255
      const bool has = lane < full;
      uint32_t mx = 0;
      const uint32_t v0[4] = {q[0].x, q[0].y, q[0].z, q[0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t e0 = (v0[j] >> 7) & 0xFFu, e1 = (v0[j] >> 23) & 0xFFu;
        mx = (e0 != 255u && e0 > mx) ? e0 : mx;
        mx = (e1 != 255u && e1 > mx) ? e1 : mx;
      }
      const uint32_t need = ((uint32_t)__popcll(__ballot(has)) + 1) / 2;
      uint32_t med = 0;
#pragma unroll
      for (int bit = 7; bit >= 0; --bit) {
        const uint32_t cand = med | (1u << bit);
        if ((uint32_t)__popcll(__ballot(has && mx >= cand)) >= need) med = cand;
      }
      lo = med > (uint32_t)kBandBelow ? med - kBandBelow : 0u;
    }
    const u16x2 lo2 = {(unsigned short)lo, (unsigned short)lo};
#pragma unroll
    for (int i = 0; i < kCountBatch; ++i) {
      if (g0 + i * kWave + lane < full) {
        const uint32_t v[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
        uint32_t out = 0;   // nonzero when a field of these 8 lies outside the band
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          atomicAdd(band + __builtin_amdgcn_ubfe(v[j], 7, 4) * kBandStride, 1u);
          atomicAdd(band + __builtin_amdgcn_ubfe(v[j], 23, 4) * kBandStride, 1u);
          out |= bits_of(as_u16x2((v[j] >> 7) & 0x00FF00FFu) - lo2) & 0xFFF0FFF0u;
        }
        if (__ballot(out != 0)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            count_outside((v[j] >> 7) & 0xFFu, lo, band, hist);
            count_outside((v[j] >> 23) & 0xFFu, lo, band, hist);
          }
        }
      }
    }
  }
  for (int i = 8 * full + lane; i < K; i += kWave) {
    const uint32_t e = (row[i] >> 7) & 0xFFu;
    atomicAdd(band + (e & (kBandBins - 1)) * kBandStride, 1u);
    count_outside(e, lo, band, hist);
  }
  // sum the lanes' band counters: lane l adds counter j = l >> 2 of lanes 16 (l & 3) .. 16 (l & 3) + 15
  // (starting at a different lane for each counter, so the reads spread over the banks), then the
  // four lanes of each counter combine; counter j holds band field lo + ((j - lo) & 15)
  {
    const int j = lane >> 2;
    const uint32_t* pf = &s_band[j][wave * kWave + (lane & 3) * 16];
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) c += pf[(i + j) & 15];
    c += __shfl_xor(c, 1, kWave);
    c += __shfl_xor(c, 2, kWave);
    const uint32_t e = lo + (((uint32_t)j - lo) & (kBandBins - 1));
    if ((lane & 3) == 0 && e >= 1u && e <= 254u) hist[e] += c;
  }
  uint32_t best;
  if (forced) {
    uint32_t b = forced[n];
    b = b < 1u ? 1u : (b > 239u ? 239u : b);
    uint32_t c = 0;
    for (uint32_t e = b; e < b + 16; ++e) c += hist[e];
    best = (c << 8) | (255u - b);
  } else {
    // P[f] = count of fields 0..f; lane l holds P[4l .. 4l + 3].  The window of base b counts
    // P[b + 15] - P[b - 1]; for b = 4l + j that takes P[4l + j - 1] (this lane, or the last of
    // lane l - 1) and P[4l + j + 15] (the last of lane l + 3 for j = 0, else lane l + 4).
    const uint4 h = reinterpret_cast<const uint4*>(hist)[lane];
    const uint32_t p0 = h.x, p1 = p0 + h.y, p2 = p1 + h.z, p3 = p2 + h.w;
    uint32_t inc = p3;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t o = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += o;
    }
    const uint32_t ex = inc - p3;   // P[4l - 1]
    const uint32_t P[4] = {ex + p0, ex + p1, ex + p2, ex + p3};
    const uint32_t up3 = __shfl_down(P[3], 3, kWave);
    const uint32_t up4_0 = __shfl_down(P[0], 4, kWave), up4_1 = __shfl_down(P[1], 4, kWave),
                   up4_2 = __shfl_down(P[2], 4, kWave);
    const uint32_t hiP[4] = {up3, up4_0, up4_1, up4_2};
    const uint32_t loP[4] = {ex, P[0], P[1], P[2]};
    best = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = 4u * lane + j;
      if (b >= 1u && b <= 239u) {
        const uint32_t key = ((hiP[j] - loP[j]) << 8) | (255u - b);
        best = key > best ? key : best;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = __shfl_xor(best, off, kWave);
      best = o > best ? o : best;
    }
  }
  if (lane == 0) {
    base[n] = (uint8_t)(255u - (best & 0xFFu));
    esc_ptr[n + 1] = (uint32_t)K - (best >> 8);
  }
}

// esc_ptr[0] = 0 and an inclusive scan of the counts in esc_ptr[1..N] (one work-group).
// The counts stream through LDS in chunks of kScanChunk: coalesced loads into LDS (all of a
// chunk's loads in flight at once); each thread sums and then scans its kScanPer contiguous
// counts there (with one pad word every 32 slots, consecutive threads' runs start 33 words
// apart, so their reads fall in distinct banks); wave shuffles and one pass over the wave
// totals give each thread its offset; coalesced stores write the chunk back, and the chunk's
// total carries into the next one.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 32;
constexpr int kScanChunk = kScanThreads * kScanPer;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kScanStride = kScanThreads + kScanThreads / 32;   // slots between counts kScanThreads apart
__device__ __forceinline__ int scan_slot(int i) { return i + (i >> 5); }
__global__ __launch_bounds__(kScanThreads) void k_scan_counts(uint32_t* __restrict__ esc_ptr, int32_t N) {
  __shared__ uint32_t buf[kScanChunk + kScanChunk / 32];
  __shared__ uint32_t wtot[kScanWaves];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  uint32_t* const bt = buf + scan_slot(t);
  uint32_t carry = 0;   // the counts of the earlier chunks
  for (int64_t c0 = 1; c0 <= (int64_t)N; c0 += kScanChunk) {
    const int len = (int)((int64_t)N + 1 - c0 < kScanChunk ? (int64_t)N + 1 - c0 : kScanChunk);
    uint32_t* const src = esc_ptr + c0;   // uniform base; 32-bit offsets below
    // slot of count k * kScanThreads + t is scan_slot(t) + k * kScanStride
    // every load is issued (past the end it rereads the last count, then counts 0), so all of
    // them are in flight together instead of one round trip each behind a branch
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, (uint32_t)len * 4u);
    uint32_t x[kScanPer];
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = k * kScanThreads + t;
      x[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (i < len ? i : len - 1), 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) bt[k * kScanStride] = k * kScanThreads + t < len ? x[k] : 0u;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) s += buf[scan_slot(t * kScanPer + j)];
    uint32_t inc = s;   // inclusive scan of the thread sums within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t o = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) wtot[wave] = inc;
    __syncthreads();
    uint32_t run = carry + (inc - s), total = 0;
    for (int w = 0; w < kScanWaves; ++w) {
      const uint32_t x = wtot[w];
      run += w < wave ? x : 0u;
      total += x;
    }
    // each thread rewrites only the slots it read
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      run += buf[scan_slot(t * kScanPer + j)];
      buf[scan_slot(t * kScanPer + j)] = run;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = k * kScanThreads + t;
      if (i < len) src[i] = bt[k * kScanStride];
    }
    carry += total;
    __syncthreads();   // buf and wtot are rewritten by the next chunk
  }
  if (t == 0) esc_ptr[0] = 0;
}

constexpr int kEmitWaves = kRowsPerBlock;   // one wave per row of a 16-row block
constexpr int kEmitThreads = kEmitWaves * kWave;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// The records of a word's two weights, each 4 bits up in its half (sign at bit 15, exponent
// offset e - b at bits 11..14, mantissa at bits 4..10), and keep: 0xFFFF in a half whose weight
// is in the window [b, b + 15], else 0 (that half's record is then 0).  bb holds b << 7 in both
// halves.  y = bits - (b << 7) (modulo 2^16) holds (e - b) << 7 plus the mantissa below the
// sign when e >= b, and wraps to bits 11..14 not all zero when e < b, so bits 11..14 of y are
// all zero exactly when 0 <= e - b <= 15; u - 1 is then the only negative value.
__device__ __forceinline__ uint32_t pair_records(uint32_t w, u16x2 bb, uint32_t& keep) {
  const u16x2 y = as_u16x2(w) - bb;
  const u16x2 u = as_u16x2(bits_of(y) & 0x78007800u);
  keep = bits_of(__builtin_bit_cast(i16x2, u - (u16x2){1, 1}) >> (i16x2){15, 15});
  return ((w & 0x80008000u) | bits_of(y << (u16x2){4, 4})) & keep;
}

// The 16 weights of chunk c of a row as 8 words (zeros past K).  Nothing is read when !live.
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ row, int32_t K, int64_t c, bool live,
                                           uint32_t w[8]) {
  uint4 a = make_uint4(0, 0, 0, 0), q = make_uint4(0, 0, 0, 0);
  if (live) {
    const int64_t rem = (int64_t)K - c * kChunkK;
    load16_bf16(row + c * kChunkK, rem >= kChunkK ? kChunkK : (int)rem, a, q);
  }
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = q.x; w[5] = q.y; w[6] = q.z; w[7] = q.w;
}

// The chunk's packed records: 16 hi bytes (rec >> 4, k ascending) and 8 lo bytes (byte i holds
// rec i in its high nibble and rec i + 4 in its low one, per half of the chunk), and the AND of
// the pairs' keep masks (all ones iff every weight of the chunk is in the window).
__device__ __forceinline__ void chunk_records(const uint32_t w[8], u16x2 bb, uint4& hi16, uint2& lo8,
                                              uint32_t& keep_all) {
  uint32_t r[8], keep[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = pair_records(w[i], bb, keep[i]);
  keep_all = keep[0] & keep[1] & keep[2] & keep[3] & keep[4] & keep[5] & keep[6] & keep[7];
  // hi: byte 1 of each half is rec >> 4
  hi16 = make_uint4(__builtin_amdgcn_perm(r[1], r[0], 0x07050301u), __builtin_amdgcn_perm(r[3], r[2], 0x07050301u),
                    __builtin_amdgcn_perm(r[5], r[4], 0x07050301u), __builtin_amdgcn_perm(r[7], r[6], 0x07050301u));
  // lo: bits 4..7 of each half are rec & 0xF; pair rec i (high nibble) with rec i + 4 (low)
  constexpr uint32_t m = 0x00F000F0u;
  uint32_t lw[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t P = (r[4 * d] & m) | ((r[4 * d + 2] >> 4) & ~m);
    const uint32_t Q = (r[4 * d + 1] & m) | ((r[4 * d + 3] >> 4) & ~m);
    lw[d] = __builtin_amdgcn_perm(Q, P, 0x06040200u);
  }
  lo8 = make_uint2(lw[0], lw[1]);
}

// Append the chunk's escapes to the row's list in ascending k (called by every lane of the wave,
// for a real row).  A lane whose chunk is whole and in the window (keep_all all ones) has none;
// when no lane has any, the wave only reads one ballot.  Otherwise each lane finds its escapes
// (the weights of its chunk, below K, whose exponent field lies outside [b, b + 15]), a wavefront
// prefix sum of their counts (one ballot per bit of the count) gives its slot after the row's
// running offset, and the offset advances by the wave's total.
__device__ __forceinline__ void chunk_escapes(const uint32_t w[8], uint32_t keep_all, bool live, int32_t K, int64_t c,
                                              uint32_t b, uint32_t& slot, uint32_t* __restrict__ esc,
                                              uint32_t num_esc) {
  const bool has = live && keep_all != 0xFFFFFFFFu;
  if (__ballot(has) == 0) return;
  uint32_t escmask = 0;
  if (has) {
    const int64_t rem = (int64_t)K - c * kChunkK;
    const int valid = rem >= kChunkK ? kChunkK : (int)rem;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t e = (w[j >> 1] >> (16 * (j & 1) + 7)) & 0xFFu;
      if (j < valid && (e < b || e > b + 15u)) escmask |= 1u << j;
    }
  }
  const uint32_t cnt = __builtin_popcount(escmask);
  uint32_t prefix = 0, total = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t mk = __ballot((cnt >> bit) & 1u);
    prefix += lanes_below(mk) << bit;
    total += (uint32_t)__popcll(mk) << bit;
  }
  uint32_t o = slot + prefix;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (escmask & (1u << j)) {
      if (o < num_esc) esc[o] = ((uint32_t)(c * kChunkK + j) << 16) | ((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      ++o;
    }
  }
  slot += total;
}

// LDS slot of row r's piece of chunk j (0..63) of an iteration, in plane order [chunk][row] with
// the row index XORed by bits of the chunk: the 16 rows' writes of one chunk and the stores'
// reads of consecutive pieces both spread over the banks.
__device__ __forceinline__ int hi_slot(int j, int r) { return j * kRowsPerBlock + (r ^ (j & 15)); }
__device__ __forceinline__ int lo_slot(int j, int r) { return j * kRowsPerBlock + (r ^ ((j >> 1) & 15)); }

// One work-group per row block; wave r encodes row 16 rb + r, lane l chunk c0 + l (16
// consecutive k).  The records of the block's 64 chunks of an iteration are staged in LDS in
// plane order and stored as one contiguous 16 KB hi run and one 8 KB lo run, every lane writing
// adjacent bytes.  Each lane loads its next chunk before encoding the current one.  The records
// are formed two weights at a time (pair_records), and a wave whose 64 chunks hold no escape
// (the common case) skips the escape compaction after one ballot.
__global__ __launch_bounds__(kEmitThreads) void k_encode_emit(
    const uint16_t* __restrict__ W, int32_t N, int32_t K, int64_t ldw, int64_t Kc,
    const uint8_t* __restrict__ base, const uint32_t* __restrict__ esc_ptr, uint8_t* __restrict__ hi,
    uint8_t* __restrict__ lo, uint32_t* __restrict__ esc, uint32_t num_esc) {
  __shared__ uint4 s_hi[kWave * kRowsPerBlock];   // [chunk][row], swizzled
  __shared__ uint2 s_lo[kWave * kRowsPerBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb = blockIdx.x;
  const int r = wave;
  const int64_t n = rb * kRowsPerBlock + r;
  const bool real = n < N;
  const uint32_t b = real ? base[n] : 1u;
  const u16x2 bb = {(unsigned short)(b << 7), (unsigned short)(b << 7)};
  uint32_t slot = real ? esc_ptr[n] : 0u;
  const uint16_t* row = W + (real ? n : 0) * ldw;
  uint32_t cur[8];
  load_chunk(row, K, lane, real && lane < Kc, cur);
  for (int64_t c0 = 0; c0 < Kc; c0 += kWave) {
    const int64_t c = c0 + lane;
    uint32_t nxt[8];
    load_chunk(row, K, c + kWave, real && c + kWave < Kc, nxt);
    uint4 h;
    uint2 l;
    uint32_t keep_all;
    chunk_records(cur, bb, h, l, keep_all);
    s_hi[hi_slot(lane, r)] = h;
    s_lo[lo_slot(lane, r)] = l;
    if (real) chunk_escapes(cur, keep_all, c < Kc, K, c, b, slot, esc, num_esc);
    __syncthreads();
    // the block's chunks c0 .. c0 + nc - 1 are contiguous in both planes
    const int64_t nc = Kc - c0 < kWave ? Kc - c0 : kWave;
    const int t = threadIdx.x;   // one 16-byte hi piece and one 8-byte lo piece per thread
    if (t < nc * kRowsPerBlock) {
      // non-temporal: the planes are not read again by this encode, and stores that bypass the
      // caches leave no dirty lines for the next kernel to write back
      const int j = t / kRowsPerBlock, rr = t % kRowsPerBlock;
      const uint4 hv = s_hi[hi_slot(j, rr)];
      const uint2 lv = s_lo[lo_slot(j, rr)];
      uint32_t* const hp = reinterpret_cast<uint32_t*>(hi + hi_offset(rb, c0, Kc, 0) + 16 * t);
      uint32_t* const lp = reinterpret_cast<uint32_t*>(lo + lo_offset(rb, c0, Kc, 0) + 8 * t);
      __builtin_nontemporal_store(hv.x, hp);
      __builtin_nontemporal_store(hv.y, hp + 1);
      __builtin_nontemporal_store(hv.z, hp + 2);
      __builtin_nontemporal_store(hv.w, hp + 3);
      __builtin_nontemporal_store(lv.x, lp);
      __builtin_nontemporal_store(lv.y, lp + 1);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
  }
}

hipError_t launch_encode_count(const uint16_t* W, int32_t N, int32_t K, int64_t ldw, const uint8_t* forced,
                               uint8_t* base, uint32_t* esc_ptr, hipStream_t stream) {
  const unsigned grid = (unsigned)((N + kCountWaves - 1) / kCountWaves);
  hipLaunchKernelGGL(k_encode_count, dim3(grid), dim3(kCountWaves * kWave), 0, stream, W, N, K, ldw, forced, base,
                     esc_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(kScanThreads), 0, stream, esc_ptr, N);
  return hipGetLastError();
}

hipError_t launch_encode_emit(const uint16_t* W, int64_t ldw, const w12_tensor* t, hipStream_t stream) {
  const int64_t Nb = num_row_blocks(t->N);
  const int64_t Kc = num_chunks(t->K);
  hipLaunchKernelGGL(k_encode_emit, dim3((unsigned)Nb), dim3(kEmitThreads), 0, stream, W, t->N, t->K, ldw, Kc,
                     t->base, t->esc_ptr, t->hi, t->lo, t->esc, (uint32_t)t->num_escapes);
  return hipGetLastError();
}

}  // namespace w12
