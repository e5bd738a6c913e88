/*
 * w12_timeline.h - measurement build of libw12 only (libw12_timeline.so, built with
 * `python -m lossless_bit_weight_encode_amd.build --timeline`; the normal libw12.so does not
 * export this).  Not part of the format or of the GEMM's contract.
 *
 * In that build every work-group of the streaming GEMM (w12_gemm with M <= 64, w12_gemm_q and
 * the grouped launch) writes 16 unsigned 64-bit values: thread 0 stamps the GPU real-time
 * counter (100 MHz) at fixed points of the kernel.  Slot meanings, per work-group w at
 * offset 16 w: 0 start, 1 prologue done, 2 / 4 first / second segment's step loop done
 * (wave 0), 3 switch to the second segment done, 5 / 8 the segment's last stage waited for,
 * 6 / 9 cross-wave reduction done, 7 / 10 partial or Y stores issued, 11 end, 12 compute-unit
 * id (__smid), 13 segments processed, 14 fixup: own partial stores complete, 15 fixup: arrival
 * counters updated.  Values of a launch persist until the next launch overwrites them; slots
 * a work-group does not reach keep older values.
 */
#ifndef W12_TIMELINE_H
#define W12_TIMELINE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Copy the first `bytes` bytes of the timeline (at most 4096 x 16 x 8) to host memory `host`
 * (synchronous).  Returns W12_OK, W12_ERR_INVALID_ARG or W12_ERR_HIP. */
int w12_timeline_copy(void *host, uint64_t bytes);

#ifdef __cplusplus
}
#endif
#endif
