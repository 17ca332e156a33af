/*
 * attn_calibrate.h -- measurement helpers of libattn.so: two kernels that
 * measure on-device ceilings a kernel's roofline fraction can also be quoted
 * against, beside the chip's published peaks.  They are not part of the
 * attention path.  Same conventions as attn.h: plain pointers to device
 * memory owned by the caller, `stream` a hipStream_t (NULL = default stream),
 * the call only enqueues work, every argument is checked on the host before
 * anything is launched, and the return value is an attn_status.
 */
#ifndef ATTN_CALIBRATE_H_
#define ATTN_CALIBRATE_H_

#include <stddef.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_calib_mfma_bf16 -- back-to-back bf16 matrix-core loop: `blocks`
 * workgroups of 4 wavefronts, each wavefront running `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 chains on register operands, i.e.
 * blocks · 4 · iters · 4 · 32768 FLOP per call.  Launched with two
 * workgroups per compute unit (blocks = 512 on 256 CUs) it keeps every
 * matrix core busy; FLOP / elapsed time is the sustained bf16 matrix rate.
 *
 *   out : [blocks · 256] fp32, written (the chains' sums, so nothing is elided)
 *
 * Errors: ATTN_ERR_NULL_PTR; ATTN_ERR_BAD_SHAPE unless 1 <= blocks <= 2^20 and
 * 1 <= iters <= 2^24; ATTN_ERR_MISALIGNED if out is not 16-byte aligned.
 */
attn_status attn_calib_mfma_bf16(float* out, int blocks, int iters, void* stream);

/*
 * attn_calib_read -- streaming read: `blocks` workgroups of 256 threads read
 * the `bytes` bytes at `buf` once, 16 bytes per thread per iteration, in a
 * grid-stride loop, and write (practically) nothing.  bytes / elapsed time is
 * the HBM read rate a plain kernel reaches (for a buffer far larger than the
 * caches).
 *
 *   buf     : `bytes` bytes, read
 *   scratch : 4096 bytes, written only in the unlikely case that a thread's
 *             XOR of what it read equals a fixed constant
 *
 * Errors: ATTN_ERR_NULL_PTR; ATTN_ERR_BAD_SHAPE unless bytes is a positive
 * multiple of 16 and 1 <= blocks <= 2^20; ATTN_ERR_MISALIGNED if buf or
 * scratch is not 16-byte aligned.
 */
attn_status attn_calib_read(const void* buf, size_t bytes, void* scratch, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CALIBRATE_H_ */
