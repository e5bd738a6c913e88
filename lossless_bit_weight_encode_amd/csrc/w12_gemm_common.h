// Building blocks shared by the two W12 GEMM kernels (the streaming kernel for few rows of X
// and the wide-tile kernel for many): buffer resources and buffer-to-LDS DMA, explicit
// memory-counter waits, LDS reads the compiler does not associate with a DMA, and host-side
// device queries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

namespace w12 {

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past any plane: reads give 0, writes are dropped
constexpr int kCachePolicySc1 = 16;             // buffer access cache policy: sc1 (device coherent)

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// The wave's index in the work-group, known to be uniform (scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int kCachePolicyNT = 2;   // the cache-policy operand's non-temporal bit (gfx950)
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kCachePolicyNT));
}
// 16 bytes per lane from the buffer into LDS: lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, 0, 0, 0);
}
// The same with the non-temporal cache policy (data read once: streamed through L2 without
// displacing what is reused).
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, 0, 0, kCachePolicyNT);
}

// The work-group's logical index.  Work-groups are handed to the 8 XCDs in turn, so physical
// block b runs on XCD b % 8; logical indices are laid out per XCD (XCD x takes a contiguous run),
// which puts the work-groups that split a tile (or share its weights) on one L2.
__device__ __forceinline__ int64_t logical_wg(int64_t b, int64_t G) {
  const int64_t x = b % 8, q = G / 8, r = G % 8;
  return x * q + (x < r ? x : r) + b / 8;
}

__device__ __forceinline__ uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)(lds_u8*)p; }

// Wait until at most N vector-memory instructions of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// A barrier without the memory fence of __syncthreads (whose release part would wait for
// every buffer-to-LDS load in flight); LDS writes are waited for explicitly before it.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

__device__ __forceinline__ uint4 lds_read_u128(uint32_t a) {
  uint4 v;
  asm volatile("ds_read_b128 %0, %1\ns_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\ns_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// A global-memory escape entry, waited for on the spot.  The compiler cannot tell the two
// escape modes apart at a cursor's later uses; a cursor register left with a load in flight
// would make it wait for all vector-memory traffic (the ring's stages included) at every step.
__device__ __forceinline__ uint32_t esc_global(const uint32_t* __restrict__ esc, uint32_t i) {
  uint32_t v;
  const uint32_t* p = esc + i;
  asm volatile("global_load_dword %0, %1, off\n"
               "s_waitcnt vmcnt(0)"
               : "=v"(v)
               : "v"(p)
               : "memory");
  return v;
}

static inline int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}

// Compute units of the current device (256 on MI355X; that value is also used when no device
// is visible, so host-only planning gives the same sizes as on the GPU).
static inline int device_cus() {
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

}  // namespace w12
