// W12 decode, load-time bit check and record unpacking.
//
// SpecPilot summary page, result bullet of section 4.1: every decoded tensor is checked bit
// for bit at load time.  News article "(1) W12": the format restores the original weights
// bit for bit, escapes from the sparse list included.
#include "w12_device.h"
#include "w12_kernels.h"

namespace w12 {

constexpr int kDecWaves = 4;
constexpr int kDecChunksPerTask = 64;   // 1024 k per wave task, 16 chunks per lane
constexpr int kDecMinChunks = 16;       // shortest task (4 chunks per lane)
constexpr int64_t kDecMinTasks = 4096;  // tasks below which they are shortened (about 4 waves per SIMD)

// A wave decodes one row block over a range of cpt chunks (64, shortened down to 16 when a
// small matrix would not give the GPU enough waves).  Lane (r, g) owns row r and the
// chunks c0 + g, c0 + g + 4, ...: one load instruction covers 4 adjacent chunks (1 KB of hi)
// and every row writes 128 contiguous bytes.  Escapes are applied through a per-lane cursor
// over the row's list (entries of the other three lanes' chunks are stepped over).
template <bool kVerify>
__global__ __launch_bounds__(kDecWaves * kWave) void k_decode(
    const uint8_t* __restrict__ base, const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
    const uint32_t* __restrict__ esc_ptr, const uint32_t* __restrict__ esc, uint32_t num_esc, int32_t N, int32_t K,
    int64_t Kc, int64_t tasks_per_rb, int64_t num_tasks, int32_t cpt, uint16_t* __restrict__ out, const uint16_t* __restrict__ ref,
    int64_t ld, unsigned long long* __restrict__ result) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t task = (int64_t)blockIdx.x * kDecWaves + wave;
  if (task >= num_tasks) return;
  const int64_t rb = task / tasks_per_rb;
  const int64_t c_begin = (task % tasks_per_rb) * cpt;
  const int64_t c_end = (c_begin + cpt < Kc) ? c_begin + cpt : Kc;
  const int64_t n = rb * kRowsPerBlock + r;
  const bool row_ok = n < N;
  const uint32_t b = row_ok ? base[n] : 1u;
  const uint32_t bb2 = base_pair(b);
  EscCursor cur;
  if (row_ok) {
    uint32_t e_lo, e_hi;
    escape_range(esc_ptr, n, num_esc, e_lo, e_hi);
    cur.idx = lower_bound_k(esc, e_lo, e_hi, (uint32_t)((c_begin + g) * kChunkK));
    cur.end = e_hi;
    cursor_load(cur, esc);
  } else {
    cur.idx = cur.end = 0;
    cur.next_k = 0xFFFFFFFFu;
    cur.next_bits = 0;
  }
  uint32_t mism = 0;
  unsigned long long first = ~0ull;
  for (int64_t c = c_begin + g; c < c_end; c += 4) {
    const uint4 h = *reinterpret_cast<const uint4*>(hi + hi_offset(rb, c, Kc, r));
    const uint2 l = *reinterpret_cast<const uint2*>(lo + lo_offset(rb, c, Kc, r));
    uint32_t d[8];
    decode16(h, l, bb2, d);
    cursor_apply(cur, esc, (uint32_t)(c * kChunkK), d);
    if (!row_ok) continue;
    const int64_t rem = (int64_t)K - c * kChunkK;
    const int valid = rem >= kChunkK ? kChunkK : (int)rem;
    const int64_t off = n * ld + c * kChunkK;
    if (!kVerify) {
      if (valid == kChunkK) {
        *reinterpret_cast<uint4*>(out + off) = make_uint4(d[0], d[1], d[2], d[3]);
        *reinterpret_cast<uint4*>(out + off + 8) = make_uint4(d[4], d[5], d[6], d[7]);
      } else {
        for (int j = 0; j < valid; ++j) out[off + j] = (uint16_t)(d[j >> 1] >> (16 * (j & 1)));
      }
    } else {
      uint4 ra, rbq;
      load16_bf16(ref + off, valid, ra, rbq);
      const uint32_t rr[8] = {ra.x, ra.y, ra.z, ra.w, rbq.x, rbq.y, rbq.z, rbq.w};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t dv = (d[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t rv = (rr[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        if (j < valid && dv != rv) {
          ++mism;
          const unsigned long long flat = (unsigned long long)n * (unsigned long long)K + c * kChunkK + j;
          first = flat < first ? flat : first;
        }
      }
    }
  }
  if (kVerify) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mism += __shfl_xor(mism, off, kWave);
      const unsigned long long o = __shfl_xor(first, off, kWave);
      first = o < first ? o : first;
    }
    if (lane == 0 && mism) {
      atomicAdd(result, (unsigned long long)mism);
      atomicMin(result + 1, first);
    }
  }
}

__global__ void k_reset_result(unsigned long long* result) {
  if (threadIdx.x == 0) {
    result[0] = 0ull;
    result[1] = ~0ull;
  }
}

// Structural check of the escape list: pointers consistent, k < K, k strictly ascending, and
// the record under each escape is the placeholder 0.  L lanes per channel (a power of two up to
// 64, from the average list length): lane j of a channel checks entries e_lo + j, + L, ...,
// each against the entry before it; lane 0 checks the pointers.
__global__ __launch_bounds__(256) void k_check_escapes(const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
                                                       const uint32_t* __restrict__ esc_ptr,
                                                       const uint32_t* __restrict__ esc, uint32_t num_esc, int32_t N,
                                                       int32_t K, int64_t Kc, int32_t lanes,
                                                       unsigned long long* __restrict__ result) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = t / lanes;
  const int j = (int)(t - n * lanes);
  uint32_t defects = 0;
  if (n < N) {
    const uint32_t a = esc_ptr[n], bnext = esc_ptr[n + 1];
    if (j == 0) {
      if (bnext < a) ++defects;
      if (bnext > num_esc) ++defects;
      if (n == 0 && a != 0) ++defects;
      if (n == N - 1 && bnext != num_esc) ++defects;
    }
    uint32_t e_lo, e_hi;
    escape_range(esc_ptr, n, num_esc, e_lo, e_hi);
    const int64_t rb = n / kRowsPerBlock;
    const int r = (int)(n % kRowsPerBlock);
    for (uint32_t i = e_lo + (uint32_t)j; i < e_hi; i += (uint32_t)lanes) {
      const uint32_t k = esc[i] >> 16;
      if (i > e_lo && k <= (esc[i - 1] >> 16)) ++defects;   // ascending within the channel
      if (k >= (uint32_t)K) {
        ++defects;
        continue;
      }
      const int64_t c = k / kChunkK;
      const int jj = (int)(k % kChunkK);
      const uint32_t hb = hi[hi_offset(rb, c, Kc, r) + jj];
      const int d = jj >> 3, i4 = jj & 7;
      const uint32_t lb = lo[lo_offset(rb, c, Kc, r) + 4 * d + (i4 & 3)];
      const uint32_t nib = (i4 < 4) ? (lb >> 4) : (lb & 0xFu);
      if (hb != 0 || nib != 0) ++defects;
    }
  }
  if (defects) atomicAdd(result, (unsigned long long)defects);
}

// Physical planes -> logical 12-bit records, one thread per (row, chunk).
__global__ __launch_bounds__(256) void k_unpack(const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
                                                int32_t N, int32_t K, int64_t Kc, uint16_t* __restrict__ rec,
                                                int64_t ldr) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = t / Kc, c = t % Kc;
  if (n >= N) return;
  const int64_t rb = n / kRowsPerBlock;
  const int r = (int)(n % kRowsPerBlock);
  const uint8_t* h = hi + hi_offset(rb, c, Kc, r);
  const uint8_t* l = lo + lo_offset(rb, c, Kc, r);
  for (int j = 0; j < kChunkK; ++j) {
    const int64_t k = c * kChunkK + j;
    if (k >= K) break;
    const int d = j >> 3, i4 = j & 7;
    const uint32_t lb = l[4 * d + (i4 & 3)];
    const uint32_t nib = (i4 < 4) ? (lb >> 4) : (lb & 0xFu);
    rec[n * ldr + k] = (uint16_t)(((uint32_t)h[j] << 4) | nib);
  }
}

static void decode_grid(const w12_tensor* t, int64_t& tasks_per_rb, int64_t& num_tasks, unsigned& grid,
                        int32_t& cpt) {
  const int64_t Kc = num_chunks(t->K);
  const int64_t nb = num_row_blocks(t->N);
  cpt = kDecChunksPerTask;
  while (cpt > kDecMinChunks && nb * ((Kc + cpt - 1) / cpt) < kDecMinTasks) cpt /= 2;
  tasks_per_rb = (Kc + cpt - 1) / cpt;
  num_tasks = num_row_blocks(t->N) * tasks_per_rb;
  grid = (unsigned)((num_tasks + kDecWaves - 1) / kDecWaves);
}

hipError_t launch_decode(const w12_tensor* t, uint16_t* out, int64_t ldo, hipStream_t stream) {
  int64_t tpr, nt;
  unsigned grid;
  int32_t cpt;
  decode_grid(t, tpr, nt, grid, cpt);
  hipLaunchKernelGGL(k_decode<false>, dim3(grid), dim3(kDecWaves * kWave), 0, stream, t->base, t->hi, t->lo,
                     t->esc_ptr, t->esc, (uint32_t)t->num_escapes, t->N, t->K, num_chunks(t->K), tpr, nt, cpt, out,
                     (const uint16_t*)nullptr, ldo, (unsigned long long*)nullptr);
  return hipGetLastError();
}

hipError_t launch_verify(const w12_tensor* t, const uint16_t* ref, int64_t ldr, unsigned long long* d_result,
                         hipStream_t stream) {
  hipLaunchKernelGGL(k_reset_result, dim3(1), dim3(64), 0, stream, d_result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t tpr, nt;
  unsigned grid;
  int32_t cpt;
  decode_grid(t, tpr, nt, grid, cpt);
  hipLaunchKernelGGL(k_decode<true>, dim3(grid), dim3(kDecWaves * kWave), 0, stream, t->base, t->hi, t->lo,
                     t->esc_ptr, t->esc, (uint32_t)t->num_escapes, t->N, t->K, num_chunks(t->K), tpr, nt, cpt,
                     (uint16_t*)nullptr, ref, ldr, d_result);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // lanes per channel: the average list length rounded up to a power of two, at most 64
  int32_t lanes = 1;
  while (lanes < 64 && (int64_t)lanes * t->N < t->num_escapes) lanes *= 2;
  const unsigned cgrid = (unsigned)(((int64_t)t->N * lanes + 255) / 256);
  hipLaunchKernelGGL(k_check_escapes, dim3(cgrid), dim3(256), 0, stream, t->hi, t->lo, t->esc_ptr, t->esc,
                     (uint32_t)t->num_escapes, t->N, t->K, num_chunks(t->K), lanes, d_result);
  return hipGetLastError();
}

hipError_t launch_unpack(const w12_tensor* t, uint16_t* rec, int64_t ldr, hipStream_t stream) {
  const int64_t Kc = num_chunks(t->K);
  const int64_t total = (int64_t)t->N * Kc;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, t->hi, t->lo, t->N, t->K,
                     Kc, rec, ldr);
  return hipGetLastError();
}

}  // namespace w12
