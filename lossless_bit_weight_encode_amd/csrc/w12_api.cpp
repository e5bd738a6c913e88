// C ABI of libw12: argument validation (host only, before any HIP call), planning and
// launches.  The declarations and their contracts are in include/w12.h.
#include <stdarg.h>
#include <stdio.h>

#include <vector>

#include "w12_device.h"
#include "w12_gemm_common.h"
#include "w12_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return W12_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxK = 65536;
constexpr int32_t kMaxM = 4096;

int check_shape(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxN) return fail(W12_ERR_UNSUPPORTED_SHAPE, "N=%lld outside 1..%lld", (long long)N, (long long)kMaxN);
  if (K < 1 || K > kMaxK) return fail(W12_ERR_UNSUPPORTED_SHAPE, "K=%lld outside 1..65536", (long long)K);
  if (N * K >= (int64_t(1) << 32)) return fail(W12_ERR_UNSUPPORTED_SHAPE, "N*K=%lld must be below 2^32", (long long)(N * K));
  // the GEMM addresses the hi plane with 32-bit buffer offsets
  if (w12::num_row_blocks(N) * w12::num_chunks(K) * w12::kHiChunkBytes >= (int64_t(1) << 32))
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "padded N x K too large for 32-bit plane offsets");
  return W12_OK;
}

// A BF16 matrix accessed with 16-byte vector loads/stores: aligned base, pitch >= cols and
// a multiple of 8 elements.
int check_bf16_matrix(const void* p, int64_t ld, int64_t cols, const char* what) {
  if (!p) return fail(W12_ERR_INVALID_ARG, "%s is NULL", what);
  if (ld < cols) return fail(W12_ERR_INVALID_ARG, "%s pitch %lld < %lld columns", what, (long long)ld, (long long)cols);
  if (!aligned(p, 16)) return fail(W12_ERR_MISALIGNED, "%s must be 16-byte aligned", what);
  if (ld % 8) return fail(W12_ERR_MISALIGNED, "%s pitch %lld must be a multiple of 8 elements", what, (long long)ld);
  return W12_OK;
}

int check_tensor(const w12_tensor* t) {
  if (!t) return fail(W12_ERR_INVALID_ARG, "tensor descriptor is NULL");
  int rc = check_shape(t->N, t->K);
  if (rc) return rc;
  if (t->layout != W12_LAYOUT_RB16_K16) return fail(W12_ERR_INVALID_ARG, "unknown layout %d", t->layout);
  if (t->reserved != 0) return fail(W12_ERR_INVALID_ARG, "reserved field must be 0");
  if (!t->base || !t->hi || !t->lo || !t->esc_ptr) return fail(W12_ERR_INVALID_ARG, "tensor has a NULL plane");
  if (t->num_escapes < 0 || t->num_escapes > (int64_t)t->N * t->K)
    return fail(W12_ERR_INVALID_ARG, "num_escapes=%lld outside 0..N*K", (long long)t->num_escapes);
  // the kernels address the escape list with 32-bit byte offsets
  if (t->num_escapes >= (int64_t(1) << 30))
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "num_escapes=%lld must be below 2^30", (long long)t->num_escapes);
  if (t->num_escapes > 0 && !t->esc) return fail(W12_ERR_INVALID_ARG, "esc is NULL with num_escapes > 0");
  if (!aligned(t->hi, 16) || !aligned(t->lo, 16)) return fail(W12_ERR_MISALIGNED, "hi and lo must be 16-byte aligned");
  if (!aligned(t->esc_ptr, 4) || (t->esc && !aligned(t->esc, 4))) return fail(W12_ERR_MISALIGNED, "esc_ptr/esc must be 4-byte aligned");
  return W12_OK;
}

// Prefix the current message with the index of the group item it concerns.
int item_fail(int code, int i) {
  char msg[sizeof(g_err)];
  snprintf(msg, sizeof(msg), "%s", g_err);
  return fail(code, "item %d: %s", i, msg);
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W12_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int w12_layout_bytes(int32_t N, int32_t K, uint64_t* hi_bytes, uint64_t* lo_bytes) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  if (!hi_bytes || !lo_bytes) return fail(W12_ERR_INVALID_ARG, "output pointer is NULL");
  const uint64_t chunks = (uint64_t)w12::num_row_blocks(N) * (uint64_t)w12::num_chunks(K);
  *hi_bytes = chunks * w12::kHiChunkBytes;
  *lo_bytes = chunks * w12::kLoChunkBytes;
  return ok();
}

int w12_encode_count(const uint16_t* W, int32_t N, int32_t K, int64_t ldw, const uint8_t* forced_base,
                     uint8_t* base, uint32_t* esc_ptr, hipStream_t stream) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  if ((rc = check_bf16_matrix(W, ldw, K, "W"))) return rc;
  if (!base || !esc_ptr) return fail(W12_ERR_INVALID_ARG, "base or esc_ptr is NULL");
  if (!aligned(esc_ptr, 4)) return fail(W12_ERR_MISALIGNED, "esc_ptr must be 4-byte aligned");
  return hip_status(w12::launch_encode_count(W, N, K, ldw, forced_base, base, esc_ptr, stream), "encode_count");
}

int w12_encode_emit(const uint16_t* W, int64_t ldw, const w12_tensor* t, hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if ((rc = check_bf16_matrix(W, ldw, t->K, "W"))) return rc;
  return hip_status(w12::launch_encode_emit(W, ldw, t, stream), "encode_emit");
}

int w12_decode(const w12_tensor* t, uint16_t* out, int64_t ldo, hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if ((rc = check_bf16_matrix(out, ldo, t->K, "out"))) return rc;
  return hip_status(w12::launch_decode(t, out, ldo, stream), "decode");
}

int w12_verify(const w12_tensor* t, const uint16_t* ref, int64_t ldr, unsigned long long* d_result,
               hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if ((rc = check_bf16_matrix(ref, ldr, t->K, "ref"))) return rc;
  if (!d_result) return fail(W12_ERR_INVALID_ARG, "d_result is NULL");
  if (!aligned(d_result, 8)) return fail(W12_ERR_MISALIGNED, "d_result must be 8-byte aligned");
  return hip_status(w12::launch_verify(t, ref, ldr, d_result, stream), "verify");
}

int w12_unpack_records(const w12_tensor* t, uint16_t* rec, int64_t ldr, hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if (!rec) return fail(W12_ERR_INVALID_ARG, "rec is NULL");
  if (ldr < t->K) return fail(W12_ERR_INVALID_ARG, "rec pitch %lld < K", (long long)ldr);
  if (!aligned(rec, 2)) return fail(W12_ERR_MISALIGNED, "rec must be 2-byte aligned");
  return hip_status(w12::launch_unpack(t, rec, ldr, stream), "unpack_records");
}

int w12_gemm_workspace_size(int32_t M, int32_t N, int32_t K, uint64_t* bytes) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  if (M < 1 || M > kMaxM) return fail(W12_ERR_UNSUPPORTED_SHAPE, "M=%d outside 1..%d", M, kMaxM);
  if (!bytes) return fail(W12_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = w12::plan_gemm(M, N, K).ws_bytes;
  return ok();
}

int w12_gemm_plan(int32_t M, int32_t N, int32_t K, w12_gemm_plan_info* info) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  if (M < 1 || M > kMaxM) return fail(W12_ERR_UNSUPPORTED_SHAPE, "M=%d outside 1..%d", M, kMaxM);
  if (!info) return fail(W12_ERR_INVALID_ARG, "info is NULL");
  const w12::GemmPlan p = w12::plan_gemm(M, N, K);
  info->path = p.path;
  info->splits = p.splits;
  info->rows_per_block = p.rb * w12::kRowsPerBlock;
  info->m_tile = p.m_tile;
  info->grid = p.grid;
  info->workspace_bytes = p.ws_bytes;
  info->counter_bytes = p.counter_bytes;
  return ok();
}

int w12_gemm_workspace_init(void* ws, uint64_t ws_bytes, hipStream_t stream) {
  if (ws_bytes == 0) return ok();
  if (!ws) return fail(W12_ERR_INVALID_ARG, "ws is NULL");
  if (!aligned(ws, 16)) return fail(W12_ERR_MISALIGNED, "ws must be 16-byte aligned");
  return hip_status(w12::init_gemm_workspace(ws, ws_bytes, stream), "gemm_workspace_init");
}

static int gemm_call(const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y, int64_t ldy, void* ws,
                     uint64_t ws_bytes, bool qpass, hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if (M < 1 || M > kMaxM) return fail(W12_ERR_UNSUPPORTED_SHAPE, "M=%d outside 1..%d", M, kMaxM);
  if ((rc = check_bf16_matrix(X, ldx, t->K, "X"))) return rc;
  if (((int64_t)M - 1) * ldx + t->K + 16 >= (int64_t(1) << 30))
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "X spans too many elements for 31-bit buffer offsets");
  if (!Y) return fail(W12_ERR_INVALID_ARG, "Y is NULL");
  if (ldy < t->N) return fail(W12_ERR_INVALID_ARG, "Y pitch %lld < N", (long long)ldy);
  if (((int64_t)M - 1) * ldy + t->N >= (int64_t(1) << 29))
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "Y spans too many elements for 31-bit buffer offsets");
  if (!aligned(Y, 4)) return fail(W12_ERR_MISALIGNED, "Y must be 4-byte aligned");
  const w12::GemmPlan p = w12::plan_gemm(M, t->N, t->K);
  if (ws_bytes < p.ws_bytes)
    return fail(W12_ERR_WORKSPACE_TOO_SMALL, "workspace %llu bytes < %llu needed", (unsigned long long)ws_bytes,
                (unsigned long long)p.ws_bytes);
  if (p.ws_bytes && !ws) return fail(W12_ERR_INVALID_ARG, "ws is NULL");
  if (ws && !aligned(ws, 16)) return fail(W12_ERR_MISALIGNED, "ws must be 16-byte aligned");
  return hip_status(w12::launch_gemm(p, X, M, ldx, t, Y, ldy, ws, qpass, stream), qpass ? "gemm_q" : "gemm");
}

int w12_gemm(const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y, int64_t ldy, void* ws,
             uint64_t ws_bytes, hipStream_t stream) {
  return gemm_call(X, M, ldx, t, Y, ldy, ws, ws_bytes, false, stream);
}

int w12_gemm_q(const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y, int64_t ldy, void* ws,
               uint64_t ws_bytes, hipStream_t stream) {
  return gemm_call(X, M, ldx, t, Y, ldy, ws, ws_bytes, true, stream);
}

int w12_gemm_noalloc(const uint16_t* X, int32_t M, int64_t ldx, const w12_tensor* t, float* Y, int64_t ldy,
                     hipStream_t stream) {
  int rc = check_tensor(t);
  if (rc) return rc;
  if (M < 1 || M > kMaxM) return fail(W12_ERR_UNSUPPORTED_SHAPE, "M=%d outside 1..%d", M, kMaxM);
  const w12::GemmPlan p = w12::plan_gemm(M, t->N, t->K);
  if (p.ws_bytes > w12::kScratchBytes)
    return fail(W12_ERR_WORKSPACE_TOO_SMALL,
                "M=%d, N=%d, K=%d needs %llu bytes of workspace, above the library's %llu-byte scratch; "
                "call w12_gemm with a workspace", M, t->N, t->K, (unsigned long long)p.ws_bytes,
                (unsigned long long)w12::kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = w12::scratch_workspace(&ws, stream);
  if (e != hipSuccess) return hip_status(e, "gemm_noalloc scratch");
  return gemm_call(X, M, ldx, t, Y, ldy, ws, w12::kScratchBytes, false, stream);
}

// Validates a group and plans it; on success fills tiles_of / upt_of and *plan.
static int group_plan(int32_t M, int32_t count, const w12_gemm_item* items, w12::GemmPlan* plan, int64_t* tiles_of,
                      int64_t* upt_of) {
  if (count < 1 || count > W12_GROUP_MAX)
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "group of %d products outside 1..%d", count, W12_GROUP_MAX);
  if (M < 1 || M > 64) return fail(W12_ERR_UNSUPPORTED_SHAPE, "grouped M=%d outside 1..64", M);
  if (!items) return fail(W12_ERR_INVALID_ARG, "items is NULL");
  std::vector<int32_t> N((size_t)count), K((size_t)count);
  for (int i = 0; i < count; ++i) {
    int rc = check_tensor(items[i].t);
    if (rc) return item_fail(rc, i);
    if (items[i].t->K % w12::kChunkK)
      return fail(W12_ERR_UNSUPPORTED_SHAPE, "item %d: K=%d is not a multiple of 16", i, items[i].t->K);
    N[i] = items[i].t->N;
    K[i] = items[i].t->K;
  }
  *plan = w12::plan_gemm_group(M, count, N.data(), K.data(), tiles_of, upt_of);
  return W12_OK;
}

int w12_gemm_group_workspace_size(int32_t M, int32_t count, const w12_gemm_item* items, uint64_t* bytes) {
  w12::GemmPlan p;
  std::vector<int64_t> tiles_of(W12_GROUP_MAX), upt_of(W12_GROUP_MAX);
  int rc = group_plan(M, count, items, &p, tiles_of.data(), upt_of.data());
  if (rc) return rc;
  if (!bytes) return fail(W12_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = p.ws_bytes;
  return ok();
}

static int gemm_group_call(int32_t M, int32_t count, const w12_gemm_item* items, void* ws, uint64_t ws_bytes,
                           bool qpass, hipStream_t stream) {
  w12::GemmPlan p;
  std::vector<int64_t> tiles_of(W12_GROUP_MAX), upt_of(W12_GROUP_MAX);
  int rc = group_plan(M, count, items, &p, tiles_of.data(), upt_of.data());
  if (rc) return rc;
  for (int i = 0; i < count; ++i) {
    const w12_gemm_item& it = items[i];
    if ((rc = check_bf16_matrix(it.X, it.ldx, it.t->K, "X"))) return item_fail(rc, i);
    if (((int64_t)M - 1) * it.ldx + it.t->K + 16 >= (int64_t(1) << 30))
      return fail(W12_ERR_UNSUPPORTED_SHAPE, "item %d: X spans too many elements for 31-bit buffer offsets", i);
    if (!it.Y) return fail(W12_ERR_INVALID_ARG, "item %d: Y is NULL", i);
    if (it.ldy < it.t->N) return fail(W12_ERR_INVALID_ARG, "item %d: Y pitch %lld < N", i, (long long)it.ldy);
    if (((int64_t)M - 1) * it.ldy + it.t->N >= (int64_t(1) << 29))
      return fail(W12_ERR_UNSUPPORTED_SHAPE, "item %d: Y spans too many elements for 31-bit buffer offsets", i);
    if (!aligned(it.Y, 4)) return fail(W12_ERR_MISALIGNED, "item %d: Y must be 4-byte aligned", i);
  }
  if (ws_bytes < p.ws_bytes)
    return fail(W12_ERR_WORKSPACE_TOO_SMALL, "workspace %llu bytes < %llu needed", (unsigned long long)ws_bytes,
                (unsigned long long)p.ws_bytes);
  if (!ws) return fail(W12_ERR_INVALID_ARG, "ws is NULL");
  if (!aligned(ws, 16)) return fail(W12_ERR_MISALIGNED, "ws must be 16-byte aligned");
  return hip_status(w12::launch_gemm_group(p, M, count, items, tiles_of.data(), upt_of.data(), ws, qpass, stream),
                    qpass ? "gemm_group_q" : "gemm_group");
}

int w12_gemm_group(int32_t M, int32_t count, const w12_gemm_item* items, void* ws, uint64_t ws_bytes,
                   hipStream_t stream) {
  return gemm_group_call(M, count, items, ws, ws_bytes, false, stream);
}

int w12_gemm_group_q(int32_t M, int32_t count, const w12_gemm_item* items, void* ws, uint64_t ws_bytes,
                     hipStream_t stream) {
  return gemm_group_call(M, count, items, ws, ws_bytes, true, stream);
}

int w12_file_write(const char* path, int32_t count, const char* const* names, const w12_tensor* host_tensors) {
  if (!path || !names || !host_tensors) return fail(W12_ERR_INVALID_ARG, "path, names or host_tensors is NULL");
  if (count < 1) return fail(W12_ERR_INVALID_ARG, "count=%d must be at least 1", count);
  for (int i = 0; i < count; ++i) {
    if (!names[i]) return fail(W12_ERR_INVALID_ARG, "names[%d] is NULL", i);
    int rc = check_tensor(&host_tensors[i]);
    if (rc) return item_fail(rc, i);
  }
  char err[256];
  if (w12::file_write(path, count, names, host_tensors, err, sizeof(err))) return fail(W12_ERR_IO, "%s", err);
  return ok();
}

int w12_file_index(const char* path, int32_t* count, w12_file_entry* entries, int32_t max_entries) {
  if (!path || !count) return fail(W12_ERR_INVALID_ARG, "path or count is NULL");
  char err[256];
  if (entries && max_entries < 0) return fail(W12_ERR_INVALID_ARG, "max_entries < 0");
  int32_t n = 0;
  if (w12::file_index(path, &n, nullptr, 0, err, sizeof(err))) return fail(W12_ERR_IO, "%s", err);
  *count = n;
  if (!entries) return ok();
  if (n > max_entries) return fail(W12_ERR_INVALID_ARG, "file holds %d tensors, room for %d", n, max_entries);
  if (w12::file_index(path, &n, entries, max_entries, err, sizeof(err))) return fail(W12_ERR_IO, "%s", err);
  return ok();
}

int w12_file_load(const char* path, int32_t count, const int32_t* which, const w12_tensor* dst, void* staging,
                  uint64_t staging_bytes, const uint16_t* const* refs, const int64_t* ldr,
                  unsigned long long* d_results, hipStream_t stream) {
  if (!path || !which || !dst) return fail(W12_ERR_INVALID_ARG, "path, which or dst is NULL");
  if (count < 1) return fail(W12_ERR_INVALID_ARG, "count=%d must be at least 1", count);
  if (!staging || staging_bytes < 512) return fail(W12_ERR_INVALID_ARG, "staging must hold at least 512 bytes");
  char err[256];
  int32_t n = 0;
  if (w12::file_index(path, &n, nullptr, 0, err, sizeof(err))) return fail(W12_ERR_IO, "%s", err);
  std::vector<w12_file_entry> idx(n);
  if (n && w12::file_index(path, &n, idx.data(), n, err, sizeof(err))) return fail(W12_ERR_IO, "%s", err);
  for (int i = 0; i < count; ++i) {
    if (which[i] < 0 || which[i] >= n) return fail(W12_ERR_INVALID_ARG, "which[%d]=%d outside 0..%d", i, which[i], n - 1);
    int rc = check_tensor(&dst[i]);
    if (rc) return item_fail(rc, i);
    const w12_file_entry& e = idx[which[i]];
    if (e.N != dst[i].N || e.K != dst[i].K || e.layout != dst[i].layout || e.num_escapes != dst[i].num_escapes)
      return fail(W12_ERR_INVALID_ARG, "item %d: descriptor does not match file entry %d (%s)", i, which[i], e.name);
    if (refs && refs[i]) {
      if (!ldr) return fail(W12_ERR_INVALID_ARG, "ldr is NULL");
      if ((rc = check_bf16_matrix(refs[i], ldr[i], dst[i].K, "ref"))) return item_fail(rc, i);
      if (!d_results) return fail(W12_ERR_INVALID_ARG, "d_results is NULL");
      if (!aligned(d_results, 8)) return fail(W12_ERR_MISALIGNED, "d_results must be 8-byte aligned");
    }
  }
  const int rc = w12::file_load(path, count, which, dst, staging, staging_bytes, refs, ldr, d_results, stream, err,
                                sizeof(err));
  if (rc == -1) return fail(W12_ERR_IO, "%s", err);
  if (rc) return fail(W12_ERR_HIP, "%s", err);
  return ok();
}

int w12_read_probe(const void* buf, uint64_t bytes, int32_t loads_per_lane, int32_t groups_per_cu, uint32_t* sink,
                   hipStream_t stream) {
  if (!buf || !sink) return fail(W12_ERR_INVALID_ARG, "buf or sink is NULL");
  // the kernel marks loads past a work-group's share with offset 2^31, which must stay past the buffer
  if (bytes < 16 || bytes % 16 || bytes > (uint64_t(1) << 31))
    return fail(W12_ERR_UNSUPPORTED_SHAPE, "bytes=%llu must be a multiple of 16 in 16..2^31", (unsigned long long)bytes);
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 && loads_per_lane != 16)
    return fail(W12_ERR_INVALID_ARG, "loads_per_lane=%d is not 1, 2, 4, 8 or 16", loads_per_lane);
  if (groups_per_cu < 1 || groups_per_cu > 16) return fail(W12_ERR_INVALID_ARG, "groups_per_cu=%d outside 1..16", groups_per_cu);
  if (!aligned(buf, 16)) return fail(W12_ERR_MISALIGNED, "buf must be 16-byte aligned");
  if (!aligned(sink, 4)) return fail(W12_ERR_MISALIGNED, "sink must be 4-byte aligned");
  const int64_t grid = (int64_t)w12::device_cus() * groups_per_cu;
  return hip_status(w12::launch_read_probe(buf, bytes, loads_per_lane, grid, sink, stream), "read_probe");
}

double w12_bits_per_weight(int32_t N, int32_t K, int64_t E) {
  if (N < 1 || K < 1 || E < 0) return -1.0;
  const double nk = (double)N * (double)K;
  return (1.5 * nk + (double)N + 4.0 * ((double)N + 1.0) + 4.0 * (double)E) * 8.0 / nk;
}

#ifdef W12_TIMELINE
#include "w12_timeline.h"
int w12_timeline_copy(void* host, uint64_t bytes) {
  if (!host) return fail(W12_ERR_INVALID_ARG, "host is NULL");
  if (bytes == 0 || bytes > (uint64_t)w12::kMaxGrid * 16 * 8)
    return fail(W12_ERR_INVALID_ARG, "bytes=%llu outside 1..%llu", (unsigned long long)bytes,
                (unsigned long long)w12::kMaxGrid * 16 * 8);
  return hip_status(w12::timeline_copy(host, bytes), "timeline_copy");
}
#endif

uint64_t w12_tensor_bytes(int32_t N, int32_t K, int64_t E) {
  if (N < 1 || K < 1 || E < 0) return 0;
  const uint64_t nk = (uint64_t)N * (uint64_t)K;
  return (12 * nk + 7) / 8 + (uint64_t)N + 4 * ((uint64_t)N + 1) + 4 * (uint64_t)E;
}

const char* w12_status_string(int status) {
  switch (status) {
    case W12_OK: return "ok";
    case W12_ERR_INVALID_ARG: return "invalid argument";
    case W12_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case W12_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case W12_ERR_HIP: return "HIP error";
    case W12_ERR_MISALIGNED: return "misaligned pointer or pitch";
    case W12_ERR_IO: return "checkpoint file error";
    default: return "unknown status";
  }
}

const char* w12_last_error(void) { return g_err; }

}  // extern "C"
