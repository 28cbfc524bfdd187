/*
 * pagedattn_bench.h -- measurement support in the same library (not part of
 * the attention path).
 *
 * The benchmark needs two plain kernels of its own: a streaming read, whose
 * bandwidth is the achievable-HBM denominator beside the published 8 TB/s,
 * and a writer that evicts L2 and the last-level cache between timed steps.
 * Both are asynchronous on `stream` (a hipStream_t; NULL = the null stream),
 * allocate nothing, and return 0, a negative status of pagedattn.h for an
 * invalid argument (nothing enqueued), or a positive hipError_t.
 */
#ifndef PAGEDATTN_BENCH_H_
#define PAGEDATTN_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` (device memory, 16-byte aligned, bytes a
 * multiple of 16) once, with coalesced 16-byte non-temporal loads: 8192
 * wavefronts, each streaming one contiguous range, 8 KB in flight each.  The XOR of every 32-bit word read is
 * XOR-ed into *sink (one device word, caller-zeroed) so that the loads are
 * live; it also lets a test check that every byte was read.
 * PA_ERR_NULL for NULL pointers, PA_ERR_SIZE for a misaligned size/address.
 */
int pa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Writes the 32-bit `value` over `bytes` bytes at `dst` (16-byte aligned,
 * a multiple of 16) with 16-byte stores.  Used to flush the caches between
 * timed steps.  Same status codes.
 */
int pa_bench_fill(void* dst, size_t bytes, uint32_t value, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BENCH_H_ */
