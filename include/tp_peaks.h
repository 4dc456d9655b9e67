/*
 * Peak probes (libtp_peaks.so): measured denominators for the roofline
 * figures that bench.py reports beside the published MI355X peaks.  They
 * are measurement tools, not part of the projector's path or its ABI
 * (include/tp.h).
 *
 * Every call launches asynchronously on `stream` (a hipStream_t as void*)
 * and returns 0, -1 for an invalid argument (nothing launched) or -3 when
 * the launch fails.  The caller owns every buffer and times the launches
 * (for instance with HIP events on the same stream).  `sink` receives a
 * value only under a condition the probes practically never meet; it must
 * hold `blocks` elements.
 */
#ifndef TP_PEAKS_H
#define TP_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of every probe. */
int tpk_threads_per_block(void);

/*
 * Read bandwidth: `blocks` workgroups read the n16 16-byte elements of the
 * device buffer `buf` (16-byte aligned) `passes` times.  The buffer is split
 * into `regions` (1 or 8) equal parts and workgroup b reads part b %
 * regions: with 8, each XCD reads its own part (workgroups are dispatched
 * round-robin over the XCDs).  Pass p starts at element p * rot of each part
 * and wraps, so a large `rot` keeps each CU's L1 from holding what the next
 * pass reads.  A buffer larger than the Infinity Cache measures HBM, one
 * that fits it but not L2 the Infinity Cache, parts that fit an XCD's L2
 * measure L2.  Bytes read = 16 * n16 * passes.  n16 and blocks must be
 * multiples of `regions`.
 */
int tpk_read(const void* buf, uint64_t n16, int64_t passes, uint64_t rot, int regions, int blocks,
             uint32_t* sink, void* stream);

/*
 * fp32 FMA rate without packed math: each thread runs 8 independent chains
 * of `iters` fused multiply-adds; flops = 16 * iters * blocks * threads.
 */
int tpk_fma(int64_t iters, int blocks, float* sink, void* stream);

/*
 * LDS 64-bit integer atomic rate: each thread adds to 8 slots of its own,
 * `iters` times (no bank conflicts, no shared address within an
 * instruction); lane operations = 8 * iters * blocks * threads.
 */
int tpk_lds_add(int64_t iters, int blocks, unsigned long long* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
