/* Ceiling kernels: what this MI355X reaches on plain HBM streams and on the
 * matrix cores, the references the hot-path kernels are measured against
 * (libtq_ceiling.so, built beside libtq.so; used by bench.py's
 * stream_ceiling workload).  They compute nothing of the method.
 *
 * All pointers are device pointers; `stream` is a hipStream_t (NULL: the
 * default stream).  Every function returns 0 on success, else the hipError_t
 * of the failed launch.  Sizes are validated on the host: a negative count
 * or a NULL pointer with work to do returns hipErrorInvalidValue (1). */
#ifndef TQ_CEILING_H
#define TQ_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The logit stream's memory traffic without its arithmetic: for each of n
 * records read 64 bytes of planes (planes + 16 i, uint32) and a 4-byte norm
 * word (norms + i), and write 4 floats, out[h * out_stride + i] for h < 4,
 * each the XOR of the record's words (so nothing can be skipped).  The
 * access pattern is the stream kernel's: 16-token tiles, a lane per 16-byte
 * word group, contiguous chunks of tiles per wave, stores of whole 32-token
 * rows.  planes 16-byte aligned, out_stride >= n. */
int tq_ceiling_logit_mix(const uint32_t* planes, const uint32_t* norms, int64_t n, float* out,
                         int64_t out_stride, void* stream);

/* The same bytes per record (64 bytes of planes and the norm word read, 4
 * floats written) in one-shot workgroups of per_block records each (a grid of
 * ceil(n / per_block) workgroups of 256 threads; thread (record t / 4, part
 * t % 4) moves 16 bytes of planes and part's float).  Small blocks keep the
 * workgroups in flight on one tight, contiguous window of memory, which is
 * the fastest mixed stream measured on this GPU (128 records per block).
 * planes 16-byte aligned, out_stride >= n, per_block >= 1. */
int tq_ceiling_logit_mix_blocks(const uint32_t* planes, const uint32_t* norms, int64_t n,
                                float* out, int64_t out_stride, int per_block, void* stream);

/* Plain device copy of `bytes` bytes (a multiple of 16; both pointers
 * 16-byte aligned), 16 bytes per lane per step. */
int tq_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Matrix-core loops: every wave of a grid of `blocks` workgroups x 4 waves
 * issues `iters` x 8 MFMAs on 4 independent accumulators, of
 * v_mfma_i32_16x16x64_i8 (kind 0, the logit stream's instruction) or
 * v_mfma_f32_32x32x16_bf16 (kind 1, the quantizer's).  out: 256 x blocks
 * floats (a sink for the accumulators).  Operations per call:
 * blocks x 4 x iters x 8 x (2 x 16 x 16 x 64 | 2 x 32 x 32 x 16). */
int tq_ceiling_mfma(int kind, int blocks, int iters, float* out, void* stream);

/* MFMA / vector-ALU co-issue: `blocks` workgroups of 8 waves (one per CU at
 * the sizes bench.py uses); waves 4-7 run v_mfma_f32_32x32x16_bf16 loops
 * (mode 0 or 2), waves 0-3 run vector work (mode 1 or 2): FMA chains
 * (kind 0) or compare / select / shift-in sequences like the quantizer's
 * code decisions (kind 1).  The time of mode 2 against modes 0 and 1 says
 * how far the two pipes overlap on one SIMD.  out: 512 x blocks floats. */
int tq_ceiling_overlap(int mode, int kind, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif
