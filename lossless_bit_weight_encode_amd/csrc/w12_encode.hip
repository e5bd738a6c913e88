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

constexpr int kCountWaves = 4;
constexpr int kCountBatch = 8;   // 16-byte loads per lane in flight before they are counted
constexpr int kHistCopies = 8;   // histogram copies per wave (lane % 8 picks one)
constexpr int kHistStride = 257; // words per copy: copies of one bin fall in different banks

// One wave per channel: LDS exponent histogram, then the best 16-wide window.  Each lane
// issues kCountBatch loads (8 KB per wave) before counting them, so a wave is not limited to
// one memory round trip per KB of its row.  A channel's exponents sit in a handful of bins,
// so the 64 lanes' atomic adds would mostly hit the same few words; eight copies of the
// histogram (summed at the end) cut those collisions eightfold.
__global__ __launch_bounds__(kCountWaves * kWave) void k_encode_count(
    const uint16_t* __restrict__ W, int32_t N, int32_t K, int64_t ldw, const uint8_t* __restrict__ forced,
    uint8_t* __restrict__ base, uint32_t* __restrict__ esc_ptr) {
  __shared__ uint32_t hist[kCountWaves][kHistCopies * kHistStride];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * kCountWaves + wave;
  uint32_t* const hw = hist[wave];
  uint32_t* const h = hw + (lane % kHistCopies) * kHistStride;   // this lane's copy
  for (int i = lane; i < kHistCopies * kHistStride; i += kWave) hw[i] = 0;
  __syncthreads();
  if (n < N) {
    const uint16_t* row = W + n * ldw;
    const int full = K / 8;   // whole 8-element groups
    for (int g0 = 0; g0 < full; g0 += kCountBatch * kWave) {
      uint4 q[kCountBatch];
#pragma unroll
      for (int i = 0; i < kCountBatch; ++i) {
        const int gi = g0 + i * kWave + lane;
        q[i] = gi < full ? *reinterpret_cast<const uint4*>(row + 8 * gi) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kCountBatch; ++i) {
        if (g0 + i * kWave + lane < full) {
          const uint32_t v[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // the word's two exponents; when they are equal (about one word in five for
            // Gaussian weights) one addition of 2 replaces two of 1, so the second addition
            // runs with fewer lanes on the contended histogram words
            const uint32_t e0 = (v[j] >> 7) & 0xFFu, e1 = (v[j] >> 23) & 0xFFu;
            atomicAdd(&h[e0], e0 == e1 ? 2u : 1u);
            if (e0 != e1) atomicAdd(&h[e1], 1u);
          }
        }
      }
    }
    for (int i = 8 * full + lane; i < K; i += kWave) atomicAdd(&h[(row[i] >> 7) & 0xFFu], 1u);
  }
  __syncthreads();
  // fold the copies into copy 0
  for (int e = lane; e < 256; e += kWave) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kHistCopies; ++i) c += hw[i * kHistStride + e];
    hw[e] = c;
  }
  __syncthreads();
  if (n < N) {
    uint32_t best;
    if (forced) {
      uint32_t b = forced[n];
      b = b < 1u ? 1u : (b > 239u ? 239u : b);
      uint32_t c = 0;
      for (uint32_t e = b; e < b + 16; ++e) c += hw[e];
      best = (c << 8) | (255u - b);
    } else {
      // key = count << 8 | (255 - b): the max key has the largest count and, among equal
      // counts, the smallest b.
      best = 0;
      for (int b = lane + 1; b <= 239; b += kWave) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) c += hw[b + e];
        const uint32_t key = (c << 8) | (255u - (uint32_t)b);
        best = key > best ? key : best;
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
}

// esc_ptr[0] = 0 and an inclusive scan of the counts in esc_ptr[1..N] (one work-group).
// The counts stream through LDS in chunks of kScanChunk: coalesced loads into LDS; each thread
// sums and then scans its kScanPer contiguous counts there (one pad word every 32 keeps those
// strided reads to 2-way bank conflicts); wave shuffles and one pass over the wave totals give
// each thread its offset; coalesced stores write the chunk back, and the chunk's total carries
// into the next one.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;
constexpr int kScanChunk = kScanThreads * kScanPer;
constexpr int kScanWaves = kScanThreads / kWave;
__device__ __forceinline__ int scan_slot(int i) { return i + (i >> 5); }
__global__ __launch_bounds__(kScanThreads) void k_scan_counts(uint32_t* __restrict__ esc_ptr, int32_t N) {
  __shared__ uint32_t buf[kScanChunk + kScanChunk / 32];
  __shared__ uint32_t wtot[kScanWaves];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  uint32_t carry = 0;   // the counts of the earlier chunks
  for (int64_t c0 = 1; c0 <= (int64_t)N; c0 += kScanChunk) {
    const int len = (int)((int64_t)N + 1 - c0 < kScanChunk ? (int64_t)N + 1 - c0 : kScanChunk);
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = k * kScanThreads + t;
      uint32_t x = 0;
      if (i < len) x = esc_ptr[c0 + i];
      buf[scan_slot(i)] = x;
    }
    __syncthreads();
    uint32_t v[kScanPer];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = buf[scan_slot(t * kScanPer + j)];
      s += v[j];
    }
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
      run += v[j];
      buf[scan_slot(t * kScanPer + j)] = run;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = k * kScanThreads + t;
      if (i < len) esc_ptr[c0 + i] = buf[scan_slot(i)];
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

// The 16 weights of chunk c of one row (a wave holds one row, lane l chunk c): their values,
// the mask of those that escape, and the packed hi bytes (16) and lo nibbles (8 bytes) of their
// records.  Lanes past the row (inactive) and rows past N (padding) give record 0 and no escape.
__device__ __forceinline__ void chunk_records(const uint16_t* __restrict__ row, int32_t K, int64_t c, bool active,
                                              bool real, uint32_t b, uint32_t v[16], uint32_t& escmask, uint4& hi16,
                                              uint2& lo8) {
  int valid = 0;
  if (active && real) {
    const int64_t rem = (int64_t)K - c * kChunkK;
    valid = rem >= kChunkK ? kChunkK : (int)rem;
    uint4 a, bq;
    load16_bf16(row + c * kChunkK, valid, a, bq);
    const uint32_t w2[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = w2[i] & 0xFFFFu;
      v[2 * i + 1] = w2[i] >> 16;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0;
  }
  uint32_t rec[16];
  escmask = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t e = (v[j] >> 7) & 0xFFu;
    const bool in = (e >= b) && (e <= b + 15u);
    const bool isreal = j < valid;
    rec[j] = (in && isreal) ? (((v[j] >> 15) << 11) | ((e - b) << 7) | (v[j] & 0x7Fu)) : 0u;
    if (isreal && !in) escmask |= 1u << j;
  }
  uint32_t hw[4], lw[2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    hw[i] = (rec[4 * i] >> 4) | ((rec[4 * i + 1] >> 4) << 8) | ((rec[4 * i + 2] >> 4) << 16) |
            ((rec[4 * i + 3] >> 4) << 24);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = ((rec[8 * d + i] & 0xFu) << 4) | (rec[8 * d + 4 + i] & 0xFu);
      x |= byte << (8 * i);
    }
    lw[d] = x;
  }
  hi16 = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  lo8 = make_uint2(lw[0], lw[1]);
}

// Append the chunk's escapes to the row's list in ascending k: every lane counts its escapes, and
// a wavefront prefix sum (one ballot per bit of the count) gives its slot after the row's running
// offset, which then advances by the wave's total.  Called by every lane of the wave.
__device__ __forceinline__ void chunk_escapes(const uint32_t v[16], uint32_t escmask, int64_t c, uint32_t& slot,
                                              uint32_t* __restrict__ esc, uint32_t num_esc) {
  const uint32_t cnt = __builtin_popcount(escmask);
  uint32_t prefix = 0, total = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t m = __ballot((cnt >> bit) & 1u);
    prefix += lanes_below(m) << bit;
    total += (uint32_t)__popcll(m) << bit;
  }
  uint32_t o = slot + prefix;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (escmask & (1u << j)) {
      if (o < num_esc) esc[o] = ((uint32_t)(c * kChunkK + j) << 16) | v[j];
      ++o;
    }
  }
  slot += total;
}

// One work-group per row block; wave r encodes row 16 rb + r, lane l chunk c0 + l (16
// consecutive k).  The records of the block's 64 chunks of an iteration are staged in LDS in
// plane order ([chunk][row][16 bytes] and [chunk][row][8 bytes]) and stored as one contiguous
// 16 KB hi run and one 8 KB lo run, every lane writing adjacent bytes.
__global__ __launch_bounds__(kEmitThreads) void k_encode_emit_blocks(
    const uint16_t* __restrict__ W, int32_t N, int32_t K, int64_t ldw, int64_t Kc,
    const uint8_t* __restrict__ base, const uint32_t* __restrict__ esc_ptr, uint8_t* __restrict__ hi,
    uint8_t* __restrict__ lo, uint32_t* __restrict__ esc, uint32_t num_esc) {
  __shared__ uint4 s_hi[kWave * kRowsPerBlock];   // [chunk][row]
  __shared__ uint2 s_lo[kWave * kRowsPerBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb = blockIdx.x;
  const int r = wave;
  const int64_t n = rb * kRowsPerBlock + r;
  const bool real = n < N;
  const uint32_t b = real ? base[n] : 1u;
  uint32_t slot = real ? esc_ptr[n] : 0u;
  const uint16_t* row = W + (real ? n : 0) * ldw;
  for (int64_t c0 = 0; c0 < Kc; c0 += kWave) {
    const int64_t c = c0 + lane;
    uint32_t v[16], escmask;
    uint4 h;
    uint2 l;
    chunk_records(row, K, c, c < Kc, real, b, v, escmask, h, l);
    s_hi[lane * kRowsPerBlock + r] = h;
    s_lo[lane * kRowsPerBlock + r] = l;
    if (real) chunk_escapes(v, escmask, c, slot, esc, num_esc);
    __syncthreads();
    // the block's chunks c0 .. c0 + nc - 1 are contiguous in both planes
    const int64_t nc = Kc - c0 < kWave ? Kc - c0 : kWave;
    const int t = threadIdx.x;   // one 16-byte hi piece and one 8-byte lo piece per thread
    if (t < nc * kRowsPerBlock) {
      *reinterpret_cast<uint4*>(hi + hi_offset(rb, c0, Kc, 0) + 16 * t) = s_hi[t];
      *reinterpret_cast<uint2*>(lo + lo_offset(rb, c0, Kc, 0) + 8 * t) = s_lo[t];
    }
    __syncthreads();
  }
}

constexpr int kEmitRowWaves = 4;

// One wave per (padded) row; lane l owns chunk c0 + l (16 consecutive k).  Records go straight
// to the hi/lo planes (16 and 8 bytes per lane, 256 and 128 bytes apart).  Used when there are
// too few row blocks to fill the GPU with block work-groups.
__global__ __launch_bounds__(kEmitRowWaves * kWave) void k_encode_emit_rows(
    const uint16_t* __restrict__ W, int32_t N, int32_t K, int64_t ldw, int64_t Np, int64_t Kc,
    const uint8_t* __restrict__ base, const uint32_t* __restrict__ esc_ptr, uint8_t* __restrict__ hi,
    uint8_t* __restrict__ lo, uint32_t* __restrict__ esc, uint32_t num_esc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * kEmitRowWaves + wave;
  if (n >= Np) return;
  const bool real = n < N;
  const int64_t rb = n / kRowsPerBlock;
  const int r = (int)(n % kRowsPerBlock);
  const uint32_t b = real ? base[n] : 1u;
  uint32_t slot = real ? esc_ptr[n] : 0u;
  const uint16_t* row = W + (real ? n : 0) * ldw;
  for (int64_t c0 = 0; c0 < Kc; c0 += kWave) {
    const int64_t c = c0 + lane;
    const bool active = c < Kc;
    uint32_t v[16], escmask;
    uint4 h;
    uint2 l;
    chunk_records(row, K, c, active, real, b, v, escmask, h, l);
    if (active) {
      *reinterpret_cast<uint4*>(hi + hi_offset(rb, c, Kc, r)) = h;
      *reinterpret_cast<uint2*>(lo + lo_offset(rb, c, Kc, r)) = l;
    }
    if (real) chunk_escapes(v, escmask, c, slot, esc, num_esc);
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
  const int64_t Np = Nb * kRowsPerBlock;
  const int64_t Kc = num_chunks(t->K);
  // Block work-groups (coalesced plane stores) when the row blocks are plenty; otherwise one wave
  // per row, which keeps more of the GPU busy.  W12_EMIT_BLOCKS = 0 / 1 forces either.
  const int force = env_int("W12_EMIT_BLOCKS", -1);
  const bool blocks = force >= 0 ? force != 0 : Nb >= 4 * (int64_t)device_cus();
  if (blocks) {
    hipLaunchKernelGGL(k_encode_emit_blocks, dim3((unsigned)Nb), dim3(kEmitThreads), 0, stream, W, t->N, t->K, ldw, Kc,
                       t->base, t->esc_ptr, t->hi, t->lo, t->esc, (uint32_t)t->num_escapes);
  } else {
    const unsigned grid = (unsigned)((Np + kEmitRowWaves - 1) / kEmitRowWaves);
    hipLaunchKernelGGL(k_encode_emit_rows, dim3(grid), dim3(kEmitRowWaves * kWave), 0, stream, W, t->N, t->K, ldw, Np,
                       Kc, t->base, t->esc_ptr, t->hi, t->lo, t->esc, (uint32_t)t->num_escapes);
  }
  return hipGetLastError();
}

}  // namespace w12
