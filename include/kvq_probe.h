/*
 * libkvq_probe -- measurement kernels that calibrate the rooflines the
 * attention and append kernels of libkvq are priced against, on the machine
 * itself ("KV Cache and autoregressive video generation", appendix section
 * [C]: measure the peak bandwidth by streaming and the peak arithmetic rate
 * by a dense product, instead of trusting a data sheet).
 *
 * These calls are measurement tools, not part of the KV-cache path.  Same
 * conventions as kvq.h: plain pointers and sizes, caller-owned device
 * memory, asynchronous on the caller's HIP stream (NULL = null stream), no
 * allocation, no synchronization.  Every argument is checked before a launch;
 * on error nothing is enqueued.
 *
 * Return value: 0 on success, 1 (invalid argument), 4 (launch failed) -- the
 * numbering of kvq_status.
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read-only HBM stream: `workgroups` workgroups of 256 threads read the
 * `bytes` bytes at `buf` once, each workgroup a contiguous share of it, with
 * 128-bit loads; each thread keeps `depth` loads (1, 2, 4, 8 or 16) in flight
 * before it consumes them.  Each workgroup stores one 32-bit word to
 * sink[workgroup] (sink: device, at least `workgroups` words) so that the
 * loads cannot be elided; nothing else is written.
 *   buf   : device, 16-byte aligned; bytes a positive multiple of 16
 * Errors: 1 for a bad size, depth, alignment or workgroup count (1 .. 2^20). */
int kvq_probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t depth,
                          uint32_t* sink, void* stream);

/* Matrix-core throughput: `workgroups` workgroups of 256 threads, each wave
 * issuing `iters` rounds of eight independent matrix instructions of one
 * kind on register operands (no memory traffic in the loop):
 *   kind 0: v_mfma_f32_16x16x32_bf16 (16384 flops each)
 *   kind 1: v_mfma_f32_16x16x32_f16  (16384 flops each)
 *   kind 2: v_mfma_i32_16x16x64_i8   (32768 integer ops each)
 * The accumulators are folded into sink[workgroup] (at least `workgroups`
 * words).  Work per call = workgroups * 4 * iters * 8 * (flops per kind).
 * Errors: 1 for a bad kind, iters < 1, or workgroup count out of range. */
int kvq_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, uint32_t* sink, void* stream);

/* An empty kernel of `workgroups` workgroups of 256 threads: the cost of a
 * launch and its dispatch, as a floor for short kernels.
 * Errors: 1 for a workgroup count out of range. */
int kvq_probe_empty(int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
