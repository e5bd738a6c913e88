// A plain streaming read of device memory: the practical HBM ceiling that the W12 GEMM's
// bandwidth is compared with.  It is a measurement aid, not part of the format.
//
// Work-group w of G reads the contiguous 16-byte elements [w n / G, (w + 1) n / G): lane t of
// the 256 takes elements beg + t + 256 i, so every load instruction of a wave reads 1 KB of
// consecutive bytes.  Each lane keeps U loads in flight: a ring of U registers, each refilled
// right after it is consumed, so the counter wait before a use leaves U - 1 loads outstanding.
// The loads use the non-temporal cache policy, the faster of the two for data read once (on
// MI355X 6.5 against 5.9 TB/s for 267 MB, 7.1 against 6.2 TB/s for 1 GiB).
// The data is folded into an XOR that is stored only if it equals a value no input here
// produces (the loads cannot be removed, and nothing is written).
#include "w12_device.h"
#include "w12_gemm_common.h"
#include "w12_kernels.h"

namespace w12 {

template <int U>
__global__ __launch_bounds__(256) void k_read_probe(const uint8_t* __restrict__ p, uint32_t bytes,
                                                    uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p, bytes);
  const uint32_t n16 = bytes / 16u;
  const uint32_t beg = (uint32_t)((uint64_t)blockIdx.x * n16 / gridDim.x);
  const uint32_t end = (uint32_t)((uint64_t)(blockIdx.x + 1) * n16 / gridDim.x);
  const uint32_t endb = end * 16u;
  constexpr uint32_t kStep = 256u * 16u;
  uint32_t off = (beg + threadIdx.x) * 16u;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v[u] = bload16_nt(r, off < endb ? off : kOutOfRange);
    off += kStep;
  }
  // every lane runs the same number of rounds (the loads past its range read zero)
  const uint32_t rounds = (end - beg + 256u * U - 1u) / (256u * U);
  uint32_t acc = 0;
  for (uint32_t i = 1; i < rounds; ++i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      v[u] = bload16_nt(r, off < endb ? off : kOutOfRange);
      off += kStep;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, int32_t loads_per_lane, int64_t grid, uint32_t* sink,
                             hipStream_t stream) {
  const dim3 g((unsigned)grid), b(256);
  const uint8_t* p = reinterpret_cast<const uint8_t*>(buf);
  const uint32_t n = (uint32_t)bytes;
  switch (loads_per_lane) {
    case 1: hipLaunchKernelGGL(k_read_probe<1>, g, b, 0, stream, p, n, sink); break;
    case 2: hipLaunchKernelGGL(k_read_probe<2>, g, b, 0, stream, p, n, sink); break;
    case 4: hipLaunchKernelGGL(k_read_probe<4>, g, b, 0, stream, p, n, sink); break;
    case 8: hipLaunchKernelGGL(k_read_probe<8>, g, b, 0, stream, p, n, sink); break;
    default: hipLaunchKernelGGL(k_read_probe<16>, g, b, 0, stream, p, n, sink); break;
  }
  return hipGetLastError();
}

}  // namespace w12
