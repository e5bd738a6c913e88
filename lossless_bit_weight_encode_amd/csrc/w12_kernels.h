// Internal launch helpers of libw12 (host side).  Arguments are validated by the C ABI
// layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w12.h"

namespace w12 {

hipError_t launch_encode_count(const uint16_t* W, int32_t N, int32_t K, int64_t ldw, const uint8_t* forced,
                               uint8_t* base, uint32_t* esc_ptr, hipStream_t stream);
hipError_t launch_encode_emit(const uint16_t* W, int64_t ldw, const w12_tensor* t, hipStream_t stream);

hipError_t launch_decode(const w12_tensor* t, uint16_t* out, int64_t ldo, hipStream_t stream);
hipError_t launch_verify(const w12_tensor* t, const uint16_t* ref, int64_t ldr, unsigned long long* d_result,
                         hipStream_t stream);
hipError_t launch_unpack(const w12_tensor* t, uint16_t* rec, int64_t ldr, hipStream_t stream);

// Every GEMM workspace starts with the same counter region, whatever the plan, so one
// initialised workspace serves any sequence of products: one arrival counter per work-group
// (a split tile counts on its first work-group's), and no launch has more work-groups.
constexpr int64_t kMaxGrid = 4096;
constexpr uint64_t kCounterBytes = (uint64_t)kMaxGrid * 4;

struct GemmPlan {
  int path;            // 1 = wavefront GEMV, 2 = MFMA tiles (streaming), 3 = wide MFMA tiles
  int splits;          // partial sums per tile (1 when a tile is never split)
  int rb;              // row blocks of 16 per tile
  int waves;           // waves per work-group (they split a segment's K range)
  int m_tile;          // rows of X per tile
  int m_tiles;         // number of m tiles
  int64_t row_groups;  // ceil(Nb / rb)
  int64_t tiles;       // row_groups * m_tiles
  int64_t upt;         // stream-K units (16 chunks) per tile
  int64_t units;       // tiles * upt
  int64_t grid;        // work-groups G (resident at once); w takes units [w U / G, (w+1) U / G)
  uint64_t counter_bytes;  // kCounterBytes: the counter region at the start of the workspace
  uint64_t partial_bytes;  // two partial tiles per work-group
  uint64_t xpad_bytes;     // the region after the partials: X copied into the workspace, padded to whole
                           // 16-k chunks (K % 16 != 0) or, for the wide tiles, rearranged into MFMA operand
                           // order; for a group past kGroupMax products, their argument blocks
  uint64_t ws_bytes;       // counters + partials + that region
};

GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K);
// The wide-tile path (many rows of X): 8 waves per work-group, tiles of 16 row blocks (256
// channels) x m_tile (128 or 256) rows of X.
constexpr int kWideWaves = 8;
constexpr int kWideRB = 16;
int wide_groups_per_cu(int m_tile);
hipError_t launch_gemm_wide(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t,
                            float* Y, int64_t ldy, void* ws, bool qpass, hipStream_t stream);

hipError_t init_gemm_workspace(void* ws, uint64_t bytes, hipStream_t stream);
// Grouped launch (several independent products of the same M, M <= 64, K % 16 == 0):
// tiles_of / upt_of receive each product's tile count and units per tile.
GemmPlan plan_gemm_group(int32_t M, int32_t count, const int32_t* N, const int32_t* K, int64_t* tiles_of,
                         int64_t* upt_of);
hipError_t launch_gemm_group(const GemmPlan& p, int32_t M, int32_t count, const w12_gemm_item* items,
                             const int64_t* tiles_of, const int64_t* upt_of, void* ws, bool qpass,
                             hipStream_t stream);
// qpass: the Q pass on the nested 8-bit view (hi plane only, escapes exact)
hipError_t launch_gemm(const GemmPlan& p, const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y,
                       int64_t ldy, void* ws, bool qpass, hipStream_t stream);

// The GEMM workspace held in the library (w12_noalloc.hip): kScratchBytes per device, its
// counter region cleared on the stream of the first call on that device.
constexpr uint64_t kScratchBytes = uint64_t(32) << 20;
hipError_t scratch_workspace(void** ws, hipStream_t stream);

#ifdef W12_TIMELINE
// Measurement build: the per-work-group timeline of the last streaming GEMM (w12_gemm.hip).
hipError_t timeline_copy(void* host, uint64_t bytes);
#endif

// Measurement aid: a plain streaming read of `bytes` bytes (w12_probe.hip).
hipError_t launch_read_probe(const void* buf, uint64_t bytes, int32_t loads_per_lane, int64_t grid, uint32_t* sink,
                             hipStream_t stream);

// Checkpoint files (host side; w12_file.cpp).  Return 0, -1 for an I/O or format error, -2
// for a HIP error, with a message in err.
uint64_t file_tensor_bytes(int32_t N, int32_t K, int64_t E);
int file_write(const char* path, int32_t count, const char* const* names, const w12_tensor* host_tensors, char* err,
               size_t errn);
int file_index(const char* path, int32_t* count, w12_file_entry* entries, int32_t max_entries, char* err,
               size_t errn);
int file_load(const char* path, int32_t count, const int32_t* which, const w12_tensor* dst, void* staging,
              uint64_t staging_bytes, const uint16_t* const* refs, const int64_t* ldr, unsigned long long* d_results,
              hipStream_t stream, char* err, size_t errn);

}  // namespace w12
