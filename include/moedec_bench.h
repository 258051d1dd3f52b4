/*
 * moedec_bench.h - measurement aids exported by libmoedec.  Not part of the
 * routed-MoE path: they give the figures the path's kernels are compared
 * against.
 *
 * Conventions as in moedec.h (device pointers, caller-owned memory, work
 * enqueued on `stream`, validated before anything is enqueued, MOEDEC_*
 * status codes).
 */
#ifndef MOEDEC_BENCH_H
#define MOEDEC_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A plain streaming read of `bytes` bytes of device memory: the achievable
 * HBM read rate on this device, the ceiling that the expert streams' rates
 * are quoted against.  The buffer is cut into `grid` contiguous stretches,
 * one per workgroup of `threads` threads; every thread reads 16-byte words
 * at consecutive addresses across its workgroup, `unroll` loads in flight
 * before any is used, and folds them with XOR.  A thread writes its fold to
 * sink[blockIdx * threads + threadIdx] only if it equals a fixed constant, so
 * the loads cannot be removed and almost nothing is written.
 *   buf    : device memory, 16-byte aligned, `bytes` readable
 *   bytes  : > 0, a multiple of 16
 *   sink   : uint32 [grid * threads], device memory (contents unspecified after)
 *   grid   : 1 .. 65536 workgroups
 *   threads: 256, 512 or 1024
 *   unroll : 4, 8 or 16
 * Errors: MOEDEC_ERR_INVALID_ARG for null or misaligned pointers and values
 * outside the ranges above.
 */
int moe_bench_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int grid, int threads, int unroll,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDEC_BENCH_H */
