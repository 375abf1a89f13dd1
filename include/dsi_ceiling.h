/*
 * dsi_ceiling.h — on-device ceilings that the indexer kernels' rooflines are
 * read against, and the plain copy that calibrates the HBM byte counters.
 *
 * Not part of the indexer path: a separate library (libdsi_ceiling.so) that
 * the benchmark loads.  The published MI355X peaks (HBM3E 8 TB/s, dense f16
 * MFMA 2.5 PFLOP/s, dense FP8 MFMA 5.0 PFLOP/s) are the roofline
 * denominators; these kernels measure what one process actually reaches:
 *   - matrix-core throughput with every operand in registers (no memory
 *     traffic, 16 independent accumulator chains per wavefront);
 *   - HBM streaming read bandwidth over a caller-sized buffer (sized well
 *     above the 256 MB Infinity Cache, so the bytes come from HBM);
 *   - the paged cache's read pattern alone: whole pages (the decode
 *     workloads' 64-token pages of 132- or 68-byte rows) read through a page
 *     table that scatters them over a pool larger than the Infinity Cache;
 *   - a plain 16-byte-per-lane copy of a known number of bytes, whose
 *     FETCH_SIZE / WRITE_SIZE counter readings give the factor between those
 *     counters and real bytes.
 *
 * Conventions: device pointers owned by the caller; each call enqueues one
 * kernel on `stream` and returns 0, or a negative dsi status (dsi.h) for
 * rejected arguments (nothing is enqueued then).
 */
#ifndef DSI_CEILING_H
#define DSI_CEILING_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSIC_API __attribute__((visibility("default")))

/* Register-only matrix-core loop.  kind 0 = v_mfma_f32_16x16x32_f16 (16,384
 * flop per instruction), kind 1 = v_mfma_scale_f32_16x16x128_f8f6f4 with FP8
 * E4M3 operands (65,536 flop per instruction), both with 16 chains per
 * wavefront; kind 2 = v_mfma_f32_32x32x16_f16 (32,768 flop per instruction)
 * with 8 chains.  Kinds 0..2 use small constant operands.  Kinds 3 and 4 are
 * kinds 0 and 2 on pseudo-random E4M3 codes (magnitudes 2 to 448, random sign
 * and mantissa) decoded to f16: the matrix cores' power depends on their
 * operands' bits, and on such data the chip runs these loops at its power
 * limit.  `workgroups` workgroups of 256 threads each run `iters` rounds of
 * one instruction per chain per wavefront, so the total is
 * workgroups * 4 * iters * chains instructions.  `sink` receives one float
 * per thread (workgroups * 256 floats) so that nothing is optimised away.
 * EINVAL: kind not 0..4, workgroups < 1, iters < 1, sink NULL. */
DSIC_API int dsic_mfma_loop(int32_t kind, int32_t workgroups, int32_t iters, float* sink, hipStream_t stream);

/* Stream-read `bytes` bytes from `src` (16-byte aligned, bytes a multiple of
 * 16) with 16-byte loads, grid-stride, and fold them into one word per thread
 * written to `sink` (workgroups * 256 uint32 = at most 4 MB).  nontemporal 1
 * sets the non-temporal hint on the loads (streaming data), 0 leaves the
 * default cache policy.  EINVAL: null pointer, bytes 0 or not a multiple of
 * 16, workgroups not 1..4096, nontemporal not 0 or 1; EALIGN: src not 16-byte
 * aligned. */
DSIC_API int dsic_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t nontemporal,
                              uint32_t* sink, hipStream_t stream);

/* Copy `bytes` bytes from `src` to `dst` (both 16-byte aligned, not
 * overlapping, bytes a multiple of 16) with 16-byte loads and stores,
 * grid-stride.  Errors as dsic_stream_read. */
DSIC_API int dsic_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, hipStream_t stream);

/* Read n_pages whole pages of page_bytes bytes, page i at pool +
 * pages[i] * block_stride (pool 16-byte aligned, pool_bytes long; page_bytes
 * a multiple of 16, at most 12288; block_stride a multiple of 16, at least
 * page_bytes), pages_per_round (4 or 8) pages per workgroup round with all
 * their loads in flight, and fold them into one word per thread written to
 * `sink` (workgroups * 256 uint32).  A page id whose page does not lie wholly
 * in the pool (negative, or past its last whole block) is read as nothing.
 * nontemporal as for dsic_stream_read.  EINVAL: null pointer, n_pages < 1,
 * pages_per_round not 4 or 8, nontemporal not 0 or 1, workgroups not
 * 1..4096, page_bytes, block_stride or pool_bytes out of range; EALIGN: pool
 * not 16-byte aligned. */
DSIC_API int dsic_paged_read(const void* pool, int64_t pool_bytes, int64_t block_stride, const int32_t* pages,
                             int32_t n_pages, int32_t page_bytes, int32_t pages_per_round, int32_t nontemporal,
                             int32_t workgroups, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSI_CEILING_H */
