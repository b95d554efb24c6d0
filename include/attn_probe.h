/*
 * attn_probe.h — measurement kernels of libattn.so: the machine ceilings the attention
 * kernels are judged against, measured on the device they run on.
 *
 * The pages set the bound that matters by the memory hierarchy (maeste.it attention-matrix
 * page, its table of bandwidth tiers: a kernel is limited by the slowest level it has to
 * stream through) and ask a measurement to state what it ran on (el-ai.com "Attenzione:
 * softmax online, riscalamento e memoria", section 5).  These entry points give the rates
 * of the units the attention kernels use, so a kernel's time can be set against what this
 * device sustains as well as against its published peak:
 *   - dense matrix-core rate, bf16 (v_mfma_f32_32x32x16_bf16) and fp8 (the 32x32x64 E4M3
 *     form the FP8 prefill uses);
 *   - the transcendental rate (v_exp_f32: one per attention weight);
 *   - HBM read bandwidth, streaming and in permuted 4 KiB pages (the paged decode's access).
 *
 * Conventions: as include/attn.h (device pointers owned by the caller, work enqueued on
 * `stream`, nothing allocated, host-visible arguments checked first, ATTN_ERR_INVALID for a
 * null pointer, a size <= 0 or more than 2^24 workgroups).  Each kernel writes a checksum the caller can verify, so
 * the work cannot be elided:
 *   - the matrix-core probes multiply blocks of ones by blocks of twos: every accumulator
 *     element ends at 32 * iters (bf16) or 128 * iters (fp8), and `out[w]` for each wave w
 *     of the grid holds the sum over one lane's 32 accumulator values, 1024 * iters or
 *     4096 * iters;
 *   - the exp probe iterates x <- 2^(-x) from 0.5 in 8 chains per lane (each x converges
 *     to the fixed point 0.6412); `out[t]` for each thread t holds the sum of its 8 values;
 *   - the read probes write, per thread of the grid, the 32-bit wrapping sum of the 32-bit
 *     words it read; their total over all threads is the wrapping sum of every word read.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of every probe (4 waves of 64). */
#define ATTN_PROBE_THREADS 256

/*
 * attn_probe_mfma — `blocks` workgroups, each wave running `iters` rounds of two
 * independent accumulation chains of the matrix-core product (fp8 = 0: bf16 32x32x16;
 * fp8 = 1: E4M3 32x32x64), two workgroups per CU.  Flops per call:
 * blocks * 4 * iters * 2 * 2 * 32 * 32 * (16 or 64).
 * out: float[blocks * 4].  iters <= 16384 (the checksum stays exact in fp32).
 */
attn_status attn_probe_mfma(int fp8, int blocks, int iters, float* out, void* stream);

/*
 * attn_probe_exp — `blocks` workgroups, each thread running `iters` rounds of 8 independent
 * v_exp_f32 chains (x <- 2^(-x), the negation a free input modifier).  Exps per call:
 * blocks * 256 * iters * 8.  out: float[blocks * 256].
 */
attn_status attn_probe_exp(int blocks, int iters, float* out, void* stream);

/*
 * attn_probe_read — reads `bytes` (a multiple of 4096) from src once, 16 bytes per lane per
 * load, four loads in flight per lane, workgroups striding over the buffer.
 * out: uint32_t[blocks * 256] (per-thread wrapping word sums).
 */
attn_status attn_probe_read(const void* src, size_t bytes, int blocks, uint32_t* out,
                            void* stream);

/*
 * attn_probe_read_pages — reads the n_pages 4 KiB pages of `pool` in the order given by
 * `order` (device int32[n_pages], each in [0, pool_pages): a precondition), one wave per
 * page at a time (four 1 KiB loads), waves striding over the order.
 * out: uint32_t[blocks * 256].
 */
attn_status attn_probe_read_pages(const void* pool, int pool_pages, const int32_t* order,
                                  int n_pages, int blocks, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
