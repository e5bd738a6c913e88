// W12 GEMM: Y[M][N] = X[M][K] . W[N][K]^T with BF16 X, W12 weights and FP32 accumulation.
//
// SpecPilot summary page, method bullet of section 4.1: the W12 GEMM decodes the records in
// registers and splits the reduction in a fixed order, so it is deterministic.  Here:
//   * every lane streams 16-k chunks of the hi/lo planes (16 + 8 bytes per row per chunk),
//     decodes them to BF16 pairs in registers (decode16) and patches the escapes of its
//     own k range through a cursor over the channel's ascending escape list;
//   * M <= 8: FP32 dot2 (v_dot2c_f32_bf16) accumulation per lane, then a fixed butterfly
//     over the 4 lanes that share a row and a fixed wave order through LDS;
//   * M >= 9: the decoded chunk is the B operand of v_mfma_f32_16x16x32_bf16 (16 rows of W
//     x 32 k), X rows padded to 16 are the A operand;
//   * the K range is cut into S slices handled by different work-groups; slice partials are
//     summed in increasing slice order by a separate kernel, never with atomics.
//
// Work decomposition.  A work-group owns `RB` row blocks (16 rows each) and one K slice; its
// W waves split the slice again and each wave's 4 lane groups split it once more, so the
// slice is cut into 4W contiguous sub-ranges of chunks.  Lane (r = lane % 16, g = lane / 16)
// of wave w handles row r of every row block for sub-range 4w + g.  The same X values are
// reused for the RB row blocks.
#include "w12_device.h"
#include "w12_kernels.h"

namespace w12 {

// Contiguous, balanced split of [0, total) into `parts`; part q is [q*total/parts, (q+1)*total/parts).
__device__ __forceinline__ int64_t split_point(int64_t total, int64_t parts, int64_t q) { return q * total / parts; }

struct RowState {
  uint32_t bb2;
  EscCursor cur;
};

__device__ __forceinline__ void init_row(RowState& rs, const uint8_t* __restrict__ base,
                                         const uint32_t* __restrict__ esc_ptr, const uint32_t* __restrict__ esc,
                                         uint32_t num_esc, int64_t n, int32_t N, uint32_t k_start) {
  if (n < N) {
    rs.bb2 = base_pair(base[n]);
    uint32_t e_lo, e_hi;
    escape_range(esc_ptr, n, num_esc, e_lo, e_hi);
    rs.cur.idx = lower_bound_k(esc, e_lo, e_hi, k_start);
    rs.cur.end = e_hi;
    cursor_load(rs.cur, esc);
  } else {
    rs.bb2 = base_pair(1);
    rs.cur.idx = rs.cur.end = 0;
    rs.cur.next_k = 0xFFFFFFFFu;
    rs.cur.next_bits = 0;
  }
}

// ------------------------------------------------------------------------------------------
// M <= 8: wavefront GEMV
// ------------------------------------------------------------------------------------------
template <int M, int RB, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_gemm_gemv(
    const uint16_t* __restrict__ X, int64_t ldx, const uint8_t* __restrict__ base, const uint8_t* __restrict__ hi,
    const uint8_t* __restrict__ lo, const uint32_t* __restrict__ esc_ptr, const uint32_t* __restrict__ esc,
    uint32_t num_esc, int32_t N, int32_t K, int64_t Kc, int64_t Nb, int32_t S, float* __restrict__ Y, int64_t ldy,
    float* __restrict__ P) {
  __shared__ float red[RB * kRowsPerBlock * M];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t rg = blockIdx.x / S;
  const int s = (int)(blockIdx.x % S);
  const int64_t nsub = (int64_t)S * WAVES * 4;
  const int64_t q = ((int64_t)s * WAVES + wave) * 4 + g;
  const int64_t c_lo = split_point(Kc, nsub, q), c_hi = split_point(Kc, nsub, q + 1);
  const int64_t iters = (Kc + nsub - 1) / nsub;

  RowState rs[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    init_row(rs[rb], base, esc_ptr, esc, num_esc, (rg * RB + rb) * kRowsPerBlock + r, N,
             (uint32_t)(c_lo * kChunkK));

  float acc[RB][M];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[rb][m] = 0.f;

  for (int64_t j = 0; j < iters; ++j) {
    const int64_t c = c_lo + j;
    if (c >= c_hi) break;
    const int64_t rem = (int64_t)K - c * kChunkK;
    const int valid = rem >= kChunkK ? kChunkK : (int)rem;
    uint32_t xv[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint4 a, b;
      load16_bf16(X + m * ldx + c * kChunkK, valid, a, b);
      xv[m][0] = a.x; xv[m][1] = a.y; xv[m][2] = a.z; xv[m][3] = a.w;
      xv[m][4] = b.x; xv[m][5] = b.y; xv[m][6] = b.z; xv[m][7] = b.w;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t rbg = rg * RB + rb;
      if (rbg >= Nb) continue;
      const uint4 h = *reinterpret_cast<const uint4*>(hi + hi_offset(rbg, c, Kc, r));
      const uint2 l = *reinterpret_cast<const uint2*>(lo + lo_offset(rbg, c, Kc, r));
      uint32_t d[8];
      decode16(h, l, rs[rb].bb2, d);
      cursor_apply(rs[rb].cur, esc, (uint32_t)(c * kChunkK), d);
#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[rb][m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d[p]),
                                                       __builtin_bit_cast(bf16x2, xv[m][p]), acc[rb][m], false);
    }
  }
  // fixed butterfly over the 4 lanes of a row: (a0 + a1) + (a2 + a3) on every lane
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[rb][m];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[rb][m] = v;
    }
  // waves in order 0, 1, ..., W-1
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w && g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float* dst = &red[(rb * kRowsPerBlock + r) * M + m];
          *dst = (w == 0) ? acc[rb][m] : *dst + acc[rb][m];
        }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < RB * kRowsPerBlock * M; i += WAVES * kWave) {
    const int row = i / M, m = i % M;
    const int64_t n = rg * RB * kRowsPerBlock + row;
    if (n >= N) continue;
    if (S == 1) Y[m * ldy + n] = red[i];
    else P[((int64_t)s * M + m) * N + n] = red[i];
  }
}

// ------------------------------------------------------------------------------------------
// M >= 9: bf16 MFMA tiles.  MB m blocks of 16 rows per work-group (m tile = 16 MB rows).
// ------------------------------------------------------------------------------------------
template <int MB, int RB, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_gemm_mfma(
    const uint16_t* __restrict__ X, int32_t M, int64_t ldx, const uint8_t* __restrict__ base,
    const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo, const uint32_t* __restrict__ esc_ptr,
    const uint32_t* __restrict__ esc, uint32_t num_esc, int32_t N, int32_t K, int64_t Kc, int64_t Nb, int32_t S,
    int32_t MT, float* __restrict__ Y, int64_t ldy, float* __restrict__ P) {
  constexpr int MTILE = MB * 16;
  __shared__ float red[RB * kRowsPerBlock * MTILE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t bid = blockIdx.x;
  const int mt = (int)(bid % MT);
  const int s = (int)((bid / MT) % S);
  const int64_t rg = bid / ((int64_t)MT * S);
  const int m0 = mt * MTILE;
  const int64_t nsub = (int64_t)S * WAVES * 4;
  const int64_t q = ((int64_t)s * WAVES + wave) * 4 + g;
  const int64_t c_lo = split_point(Kc, nsub, q), c_hi = split_point(Kc, nsub, q + 1);
  const int64_t iters = (Kc + nsub - 1) / nsub;

  RowState rs[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    init_row(rs[rb], base, esc_ptr, esc, num_esc, (rg * RB + rb) * kRowsPerBlock + r, N,
             (uint32_t)(c_lo * kChunkK));

  f32x4 acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t j = 0; j < iters; ++j) {
    const int64_t c = c_lo + j;
    const bool cv = c < c_hi;   // lanes of a wave may own sub-ranges one chunk apart in length
    const int64_t rem = (int64_t)K - c * kChunkK;
    const int valid = cv ? (rem >= kChunkK ? kChunkK : (int)rem) : 0;
    uint4 xa[MB], xb[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + r;
      if (m < M && valid > 0) {
        load16_bf16(X + (int64_t)m * ldx + c * kChunkK, valid, xa[mb], xb[mb]);
      } else {
        xa[mb] = make_uint4(0, 0, 0, 0);
        xb[mb] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t rbg = rg * RB + rb;
      if (rbg >= Nb) continue;
      uint32_t d[8];
      if (cv) {
        const uint4 h = *reinterpret_cast<const uint4*>(hi + hi_offset(rbg, c, Kc, r));
        const uint2 l = *reinterpret_cast<const uint2*>(lo + lo_offset(rbg, c, Kc, r));
        decode16(h, l, rs[rb].bb2, d);
        cursor_apply(rs[rb].cur, esc, (uint32_t)(c * kChunkK), d);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = 0;
      }
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(d[4], d[5], d[6], d[7]));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mb]), b0, acc[rb][mb], 0,
                                                              0, 0);
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xb[mb]), b1, acc[rb][mb], 0,
                                                              0, 0);
      }
    }
  }
  // lane (r, g) holds C[m = 4g + i][n = r] of every (rb, mb) tile; waves add in order 0..W-1
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = &red[(rb * kRowsPerBlock + r) * MTILE + mb * 16 + 4 * g + i];
            *dst = (w == 0) ? acc[rb][mb][i] : *dst + acc[rb][mb][i];
          }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < RB * kRowsPerBlock * MTILE; i += WAVES * kWave) {
    const int row = i / MTILE, ml = i % MTILE;
    const int64_t n = rg * RB * kRowsPerBlock + row;
    const int m = m0 + ml;
    if (n >= N || m >= M) continue;
    if (S == 1) Y[(int64_t)m * ldy + n] = red[i];
    else P[((int64_t)s * M + m) * N + n] = red[i];
  }
}

// Y[m][n] = P[0][m][n] + P[1][m][n] + ... + P[S-1][m][n], summed left to right.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ P, int32_t S, int32_t M, int32_t N,
                                                       float* __restrict__ Y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t mn = (int64_t)M * N;
  if (i >= mn) return;
  float v = P[i];
  for (int s = 1; s < S; ++s) v += P[(int64_t)s * mn + i];
  const int64_t m = i / N, n = i % N;
  Y[m * ldy + n] = v;
}

// ------------------------------------------------------------------------------------------
// Planning and launch
// ------------------------------------------------------------------------------------------
constexpr int kRB = 4;
constexpr int kWaves = 4;
constexpr int kTargetGroups = 1024;   // 4 work-groups of 4 waves per CU on 256 CUs
constexpr int kMinChunksPerLane = 2;

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
  const int64_t base_groups = p.row_groups * p.m_tiles;
  int64_t s = (kTargetGroups + base_groups - 1) / base_groups;
  const int64_t s_max = Kc / (int64_t)(p.waves * 4 * kMinChunksPerLane);
  if (s > s_max) s = s_max;
  if (s < 1) s = 1;
  p.splits = (int)s;
  p.grid = base_groups * p.splits;
  p.ws_bytes = p.splits > 1 ? (uint64_t)p.splits * (uint64_t)M * (uint64_t)N * sizeof(float) : 0;
  return p;
}

template <int M>
static void launch_gemv_m(const GemmPlan& p, const uint16_t* X, int64_t ldx, const w12_tensor* t, float* Y,
                          int64_t ldy, float* P, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_gemv<M, kRB, kWaves>), dim3((unsigned)p.grid), dim3(kWaves * kWave), 0, stream, X, ldx,
                     t->base, t->hi, t->lo, t->esc_ptr, t->esc, (uint32_t)t->num_escapes, t->N, t->K,
                     num_chunks(t->K), num_row_blocks(t->N), p.splits, Y, ldy, P);
}

template <int MB>
static void launch_mfma_mb(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t,
                           float* Y, int64_t ldy, float* P, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_mfma<MB, kRB, kWaves>), dim3((unsigned)p.grid), dim3(kWaves * kWave), 0, stream, X, M,
                     ldx, t->base, t->hi, t->lo, t->esc_ptr, t->esc, (uint32_t)t->num_escapes, t->N, t->K,
                     num_chunks(t->K), num_row_blocks(t->N), p.splits, p.m_tiles, Y, ldy, P);
}

hipError_t launch_gemm(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y,
                       int64_t ldy, void* ws, hipStream_t stream) {
  float* P = reinterpret_cast<float*>(ws);
  if (p.path == 1) {
    switch (M) {
      case 1: launch_gemv_m<1>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 2: launch_gemv_m<2>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 3: launch_gemv_m<3>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 4: launch_gemv_m<4>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 5: launch_gemv_m<5>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 6: launch_gemv_m<6>(p, X, ldx, t, Y, ldy, P, stream); break;
      case 7: launch_gemv_m<7>(p, X, ldx, t, Y, ldy, P, stream); break;
      default: launch_gemv_m<8>(p, X, ldx, t, Y, ldy, P, stream); break;
    }
  } else {
    switch (p.m_tile / 16) {
      case 1: launch_mfma_mb<1>(p, X, M, ldx, t, Y, ldy, P, stream); break;
      case 2: launch_mfma_mb<2>(p, X, M, ldx, t, Y, ldy, P, stream); break;
      case 3: launch_mfma_mb<3>(p, X, M, ldx, t, Y, ldy, P, stream); break;
      default: launch_mfma_mb<4>(p, X, M, ldx, t, Y, ldy, P, stream); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    const int64_t mn = (int64_t)M * t->N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream, P, p.splits, M,
                       t->N, Y, ldy);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace w12
