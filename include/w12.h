/*
 * w12.h - C ABI of libw12: the W12 lossless 12-bit BF16 weight format on MI355X (gfx950).
 *
 * The format (SpecPilot, arXiv 2611.02501; summary page, method bullet of section 4.1, and
 * the news article part "(1) W12"): a 12-bit record per BF16 weight,
 *   sign (1 bit) | exponent minus the channel's window base (4 bits, a window of 16
 *   binades per output channel) | top 7 mantissa bits,
 * plus an exact side list (the escapes) for weights the record cannot hold: exponents
 * outside the window, zeros, subnormals and inf/NaN.  Loading compares each decoded tensor
 * with its source bit for bit (summary page, result bullet of section 4.1); the GEMM decodes
 * records in registers and reduces its K split in a fixed order, so its bits repeat from run
 * to run (method bullet of section 4.1).
 *
 * Logical format (what every result is defined on):
 *   base[n]        window base exponent field b_n in 1..239; the window is [b_n, b_n+15].
 *                  b_n is the smallest b that maximises the number of in-window weights.
 *   rec[n][k]      (s << 11) | ((e - b_n) << 7) | m for in-window weights, 0 at escapes.
 *   esc_ptr[N+1]   exclusive prefix sum of per-channel escape counts (esc_ptr[0] = 0).
 *   esc[E]         (k << 16) | bf16_bits, channel after channel, ascending k in a channel.
 *
 * Physical layout W12_LAYOUT_RB16_K16 (this library's choice; w12_unpack_records gives the
 * logical records back).  Rows are grouped in row blocks of 16 (Nb = ceil(N/16)) and k in
 * chunks of 16 (Kc = ceil(K/16)); rows >= N and k >= K are padding with record 0.
 *   hi: uint8 [Nb][Kc][16 rows][16]  byte j of row r = rec >> 4 = s | off(4) | m[6:4]
 *       (also the nested 8-bit view of each weight).
 *   lo: uint8 [Nb][Kc][16 rows][8]   the low mantissa nibbles rec & 0xF of the 16 weights:
 *       byte 4d+i (d = 0,1; i = 0..3) holds weight 8d+i in its high nibble and weight
 *       8d+4+i in its low nibble.
 *
 * Conventions for every call:
 *   - All pointers are device pointers owned by the caller; the library never allocates
 *     and never frees.  BF16 data is passed as uint16_t bit patterns.
 *   - Every call that takes a stream only validates on the host and enqueues kernels on
 *     that stream; it returns before the GPU work finishes.  No call synchronises.
 *   - Return value: W12_OK (0) or a negative W12_ERR_* code.  Arguments are validated
 *     before any HIP call; on an error nothing is enqueued.  w12_last_error() gives a
 *     message for the last failing call of the calling thread.
 *   - Row pitches (ldw, ldx, ldo, ldr, ldy) are in elements.  BF16 matrices read or
 *     written with vector accesses (W, X, decode output, verify reference) need a
 *     16-byte aligned base pointer and a pitch that is a multiple of 8 elements.
 *   - Shapes: 1 <= N <= 2^24, 1 <= K <= 65536 (k fits the 16-bit field of an escape
 *     entry), N*K < 2^32 (escape counts are 32-bit); 1 <= M <= 4096 for the GEMM, whose
 *     X and Y must each span fewer than 2^29 elements ((M-1)*pitch + row length).
 */
#ifndef W12_H
#define W12_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W12_OK 0
#define W12_ERR_INVALID_ARG (-1)          /* null pointer, bad pitch, bad descriptor        */
#define W12_ERR_UNSUPPORTED_SHAPE (-2)    /* N, K or M outside the supported ranges          */
#define W12_ERR_WORKSPACE_TOO_SMALL (-3)  /* ws_bytes below w12_gemm_workspace_size          */
#define W12_ERR_HIP (-4)                  /* a HIP runtime call or kernel launch failed      */
#define W12_ERR_MISALIGNED (-5)           /* a vector-accessed pointer or pitch is unaligned */
#define W12_ERR_IO (-6)                   /* a checkpoint file could not be read or written  */

#define W12_LAYOUT_RB16_K16 1

/* Descriptor of an encoded tensor.  All arrays are device memory owned by the caller. */
typedef struct w12_tensor {
  int32_t N, K;          /* logical shape of W[N][K]                                     */
  int32_t layout;        /* W12_LAYOUT_RB16_K16                                          */
  int32_t reserved;      /* must be 0                                                    */
  int64_t num_escapes;   /* E = esc_ptr[N], below 2^30                                   */
  uint8_t *base;         /* [N]                                                          */
  uint8_t *hi;           /* [w12_layout_bytes().hi_bytes]                                */
  uint8_t *lo;           /* [w12_layout_bytes().lo_bytes]                                */
  uint32_t *esc_ptr;     /* [N+1]                                                        */
  uint32_t *esc;         /* [E] (may be NULL when E == 0)                                */
} w12_tensor;

/* Sizes of the hi and lo planes of the physical layout for W[N][K].  Host only. */
int w12_layout_bytes(int32_t N, int32_t K, uint64_t *hi_bytes, uint64_t *lo_bytes);

/*
 * Encode pass 1 (window choice, summary page method bullet of section 4.1; news article
 * "(1) W12": exponents cluster within a channel).  For every channel n of the BF16 matrix
 * W (row pitch ldw) computes base[n] (or copies forced_base[n] when forced_base is not
 * NULL - a test hook; each value must be in 1..239) and writes
 *   esc_ptr[0] = 0, esc_ptr[n+1] = sum_{i<=n} (K - in-window count of channel i).
 * The caller reads E = esc_ptr[N] back to size esc[] before w12_encode_emit.
 * forced_base values outside 1..239 are clamped into range by the kernel (the host
 * cannot inspect device memory without synchronising).
 */
int w12_encode_count(const uint16_t *W, int32_t N, int32_t K, int64_t ldw,
                     const uint8_t *forced_base, uint8_t *base, uint32_t *esc_ptr,
                     hipStream_t stream);

/*
 * Encode pass 2 (records and escape list, summary page method bullet of section 4.1).
 * Reads W and t->base / t->esc_ptr written by w12_encode_count and writes t->hi, t->lo
 * (padding included) and t->esc.  Escapes of a channel are compacted in ascending k with
 * wavefront prefix sums.  t->num_escapes must equal esc_ptr[N].
 */
int w12_encode_emit(const uint16_t *W, int64_t ldw, const w12_tensor *t, hipStream_t stream);

/*
 * Full-tensor decode (summary page result bullet of section 4.1: decoded tensors are the
 * original weights bit for bit).  Writes out[n][k] (row pitch ldo) for n < N, k < K.
 * The escape list must be well formed (ascending k < K per channel); w12_verify checks it.
 */
int w12_decode(const w12_tensor *t, uint16_t *out, int64_t ldo, hipStream_t stream);

/*
 * Load-time bit-for-bit check (summary page result bullet of section 4.1).  Decodes t and
 * compares with ref (row pitch ldr).  Writes, on the device,
 *   d_result[0] = number of positions (n,k) whose decoded bits differ from ref[n][k]
 *                 plus the number of malformed escape entries (k >= K, k not above the k
 *                 of the entry before it in its channel, non-zero record under an escape) plus
 *                 the number of inconsistent pointers (esc_ptr[0] != 0, a decreasing
 *                 step, esc_ptr[N] != num_escapes);
 *   d_result[1] = smallest flat index n*K + k of a differing position, or
 *                 0xFFFFFFFFFFFFFFFF if there is none.
 * d_result must point to 2 device uint64 values; the call resets them first.
 */
int w12_verify(const w12_tensor *t, const uint16_t *ref, int64_t ldr,
               unsigned long long *d_result, hipStream_t stream);

/* Test aid: writes the logical 12-bit records rec[n][k] (row pitch ldr, uint16) of the
 * physical planes, so parity with an implementation of the logical format does not
 * depend on this library's layout. */
int w12_unpack_records(const w12_tensor *t, uint16_t *rec, int64_t ldr, hipStream_t stream);

/* Bytes of device workspace w12_gemm needs for M rows of X against W[N][K]. Host only.
 * The workspace starts with a 16 KB region of 32-bit arrival counters (split-K bookkeeping;
 * the same region for every plan, single or grouped) followed by the FP32 slice partials
 * and, where the plan needs it, a copy of X that the call writes itself: for M >= 65 X
 * rearranged into the matrix cores' operand order, otherwise, for K % 16 != 0, X padded
 * with zeros to whole 16-k chunks.
 * The size follows the plan, so a change of W12_GEMV_MAX_M between sizing and calling can
 * make the workspace too small (reported as W12_ERR_WORKSPACE_TOO_SMALL). */
int w12_gemm_workspace_size(int32_t M, int32_t N, int32_t K, uint64_t *bytes);

/* Zero-fill a GEMM workspace of ws_bytes bytes on `stream`.  Call it once after allocating
 * the workspace: w12_gemm needs the counter region to be zero on entry and leaves it zero
 * when it completes, so the workspace can then serve any sequence of w12_gemm calls on one
 * stream.  Calls that overlap in time on one workspace race. */
int w12_gemm_workspace_init(void *ws, uint64_t ws_bytes, hipStream_t stream);

/*
 * Y[m][n] = sum_k X[m][k] * W[n][k] for m < M, n < N (summary page method bullet of
 * section 4.1: the GEMM decodes W12 records in registers and reduces in a fixed order).
 * X: BF16 [M][ldx]; Y: FP32 [M][ldy], every Y[m][n] (n < N) is written.  Accumulation is
 * FP32; the result is within 2^-12 * sum_k |x w| of the exact sum and bitwise identical
 * from run to run on the same device for the same (M, N, K).  M <= 2 runs a wavefront
 * GEMV (FP32 dot2 products and a fixed-order wavefront reduction), larger M runs bf16 MFMA
 * tiles; the environment variable W12_GEMV_MAX_M (0..8, read at each call) moves that
 * boundary, and W12_MAX_GRID (read at each call) caps the number of work-groups.  The K range may be split over several work-groups;
 * the last one to finish a tile sums the slice partials in increasing slice order (no
 * floating-point atomics).  ws: device workspace of at least w12_gemm_workspace_size bytes,
 * initialised once with w12_gemm_workspace_init (only its counter region must be zero; the
 * partial region may hold anything on entry).
 */
int w12_gemm(const uint16_t *X, int32_t M, int64_t ldx, const w12_tensor *t,
             float *Y, int64_t ldy, void *ws, uint64_t ws_bytes, hipStream_t stream);

/*
 * The Q pass of two-level verification (news article, two-level verification part: the
 * first pass verifies at low precision with the 8-bit weight view nested in W12 and accepts
 * nothing).  Y = X . Wq^T, where Wq is W with every in-window weight read through the
 * record's top byte (sign, exponent offset, three mantissa bits), i.e. truncated toward zero
 * to four significant bits, and every escaped weight exact.  Only the hi plane of the records
 * is read (1 byte per weight).  Same arguments, layouts, workspace, errors, tolerance (against
 * the FP64 product with Wq) and run-to-run determinism as w12_gemm.
 */
int w12_gemm_q(const uint16_t *X, int32_t M, int64_t ldx, const w12_tensor *t,
               float *Y, int64_t ldy, void *ws, uint64_t ws_bytes, hipStream_t stream);

/*
 * w12_gemm for callers that cannot allocate device memory: code under stream capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * layouts, errors, tolerance and result as w12_gemm: Y is bitwise identical to w12_gemm's for
 * the same operands.  The workspace is a 32 MiB array held by the library on each device (kept
 * until the process ends); it covers every M <= 64 (the streaming tiles) with K <= 64,000 at the
 * default launch shape, and a product whose plan needs more is rejected with W12_ERR_WORKSPACE_TOO_SMALL (call w12_gemm
 * with a workspace instead).  Nothing is allocated: the first call on a device looks up the
 * array's address and clears its counter region on `stream` (a kernel launch); every call
 * leaves it clear.  All calls on one device share the one array, so calls that overlap in time
 * on one device (on different streams or host threads) race.
 */
int w12_gemm_noalloc(const uint16_t *X, int32_t M, int64_t ldx, const w12_tensor *t,
                     float *Y, int64_t ldy, hipStream_t stream);

/*
 * Grouped launch: several independent products of the same M in one launch (summary page
 * method bullet of section 4.1: the W12 GEMM is a stream-K GEMM whose split is reduced in a
 * fixed order).  items[i] asks for Y_i = X_i . W_i^T exactly as w12_gemm would (same operand
 * layouts, pitches and alignment rules, the same tolerance); the launch streams the W12 records
 * of all count products under one stream-K schedule over their concatenated work units, so the
 * pipeline fill, the tail and the split-K fixups are paid once per launch rather than once per
 * product.  Each Y_i is bitwise identical from run to run for the same (M, shapes, order of the
 * items), though not in general bitwise equal to w12_gemm's result (the K split points differ).
 * The products must not depend on one another: no Y_i may overlap any X_j or W_j of the group.
 * Limits: 1 <= count <= W12_GROUP_MAX; 1 <= M <= 64; every K a multiple of 16.  Outside them
 * the call returns W12_ERR_UNSUPPORTED_SHAPE.  items and the descriptors they point to are host
 * memory read during the call only.  ws: at least w12_gemm_group_workspace_size bytes,
 * initialised once with w12_gemm_workspace_init (counters at its start; every call leaves them
 * zero).  Up to W12_GROUP_INLINE products travel in the kernel arguments; a larger group (a
 * whole model, say) first stores its per-product argument blocks (about 200 bytes each) at the
 * end of the workspace, with one small kernel per W12_GROUP_INLINE products on `stream`, so the
 * workspace of such a group carries that region too.  W12_GEMV_MAX_M, W12_GROUPS_PER_CU and
 * W12_MAX_GRID apply as for w12_gemm.
 */
#define W12_GROUP_MAX 1024
#define W12_GROUP_INLINE 8
typedef struct w12_gemm_item {
  const uint16_t *X;     /* BF16 [M][ldx], device                                          */
  int64_t ldx;
  const w12_tensor *t;   /* host descriptor of W_i (device planes)                         */
  float *Y;              /* FP32 [M][ldy], device                                          */
  int64_t ldy;
} w12_gemm_item;
int w12_gemm_group_workspace_size(int32_t M, int32_t count, const w12_gemm_item *items, uint64_t *bytes);
int w12_gemm_group(int32_t M, int32_t count, const w12_gemm_item *items, void *ws, uint64_t ws_bytes,
                   hipStream_t stream);
/* The Q pass (as w12_gemm_q) of every product of a group, in one launch. */
int w12_gemm_group_q(int32_t M, int32_t count, const w12_gemm_item *items, void *ws, uint64_t ws_bytes,
                     hipStream_t stream);

/* How w12_gemm will run (M, N, K).  Host only. */
typedef struct w12_gemm_plan_info {
  int32_t path;              /* 1 = wavefront GEMV, 2 = MFMA tiles, 3 = wide MFMA tiles  */
  int32_t splits;            /* most K slices (partial sums) of one output tile          */
  int32_t rows_per_block;    /* rows of W per work-group tile                            */
  int32_t m_tile;            /* rows of X per work-group tile                            */
  int64_t grid;              /* work-groups launched                                     */
  uint64_t workspace_bytes;  /* == w12_gemm_workspace_size                               */
  uint64_t counter_bytes;    /* leading bytes of the workspace holding the counters (the
                                same for every plan)                                      */
} w12_gemm_plan_info;
int w12_gemm_plan(int32_t M, int32_t N, int32_t K, w12_gemm_plan_info *info);

/*
 * W12 checkpoint files (summary page, result bullet of section 4.1: converted layers are
 * checked bit for bit when they are loaded).  A file holds named encoded tensors in the
 * physical layout above: a 64-byte header (magic "W12CKPT1", version 1, tensor count), one
 * 128-byte index entry per tensor, then per tensor its base, esc_ptr, esc, hi and lo arrays,
 * each starting on a 256-byte boundary.  Integers are little-endian.
 */
typedef struct w12_file_entry {
  char name[64];         /* NUL-terminated (at most 63 characters are stored)           */
  int32_t N, K;
  int32_t layout;        /* W12_LAYOUT_RB16_K16                                          */
  int32_t reserved;
  int64_t num_escapes;
  uint64_t offset;       /* file offset of the tensor's data                             */
  uint64_t bytes;        /* bytes of the tensor's data (sections and their padding)      */
} w12_file_entry;

/* Write count tensors to path (created or truncated).  Every array of host_tensors[i] is HOST
 * memory (copy the planes back from the device first); names[i] are C strings.  Synchronous;
 * W12_ERR_IO on a failed open or write. */
int w12_file_write(const char *path, int32_t count, const char *const *names, const w12_tensor *host_tensors);

/* Read the index of path: *count receives the number of tensors; when entries is not NULL the
 * first *count entries are written (W12_ERR_INVALID_ARG if *count > max_entries).  Synchronous. */
int w12_file_index(const char *path, int32_t *count, w12_file_entry *entries, int32_t max_entries);

/*
 * Streamed load.  For i < count, copies tensor which[i] of the file into the device arrays of
 * dst[i] (N, K, layout and num_escapes must equal the index entry; the caller sizes the arrays
 * from the entry).  The file is read on the calling thread in pieces of staging_bytes / 2
 * into alternating halves of `staging` (pinned host memory of at least 512 bytes), each piece
 * copied to the device on `stream`; a half is refilled only after its previous copy has
 * completed.  When refs is not NULL and refs[i] is not NULL, the load-time check of dst[i]
 * against the BF16 matrix refs[i] (device, row pitch ldr[i]) is enqueued on `stream` right
 * after the tensor's copies, with w12_verify's semantics, into d_results[2i], d_results[2i+1]
 * (device; 2*count values).  The call returns once every copy has been enqueued and the
 * staging buffer is no longer read; the checks may still be running.  Creates and destroys
 * two HIP events; allocates no memory.  W12_ERR_IO on a read failure or a malformed file.
 */
int w12_file_load(const char *path, int32_t count, const int32_t *which, const w12_tensor *dst,
                  void *staging, uint64_t staging_bytes, const uint16_t *const *refs, const int64_t *ldr,
                  unsigned long long *d_results, hipStream_t stream);

/*
 * Measurement aid (not part of the format): a plain streaming read of buf[0, bytes) by
 * groups_per_cu 256-thread work-groups per compute unit, each reading a contiguous share with
 * 16-byte loads (1 KB of consecutive bytes per wave instruction) and keeping loads_per_lane
 * (1, 2, 4, 8 or 16) loads in flight per lane.  It gives the practical HBM read ceiling that the
 * GEMM's bytes moved per second are compared with.  buf: device, 16-byte aligned; bytes: a
 * multiple of 16, 16 <= bytes <= 2^31; groups_per_cu: 1..16; sink: device, at least
 * groups_per_cu * (compute units) uint32 values, never written in practice (the loaded data
 * is folded into a value that is stored only if it equals a fixed constant).
 */
int w12_read_probe(const void *buf, uint64_t bytes, int32_t loads_per_lane, int32_t groups_per_cu,
                   uint32_t *sink, hipStream_t stream);

/* Stored bits per weight: (1.5*N*K + N + 4*(N+1) + 4*E) * 8 / (N*K).  -1 for N < 1, K < 1
 * or E < 0. */
double w12_bits_per_weight(int32_t N, int32_t K, int64_t E);

/* Bytes of the logical format for W[N][K] with E escapes: ceil(12 N K / 8) record bytes, one
 * base byte per channel, (N + 1) 4-byte escape pointers and 4 bytes per escape.  0 for N < 1,
 * K < 1 or E < 0.  (The device planes are padded to whole 16 x 16 chunks: w12_layout_bytes.) */
uint64_t w12_tensor_bytes(int32_t N, int32_t K, int64_t E);

const char *w12_status_string(int status);
const char *w12_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W12_H */
