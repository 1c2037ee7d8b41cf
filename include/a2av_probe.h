/*
 * a2av_probe.h -- probes of the MI355X library: the rates that the copy
 * kernel's own memory instructions reach on the device when they only read,
 * only write, or copy, and the cost of a cooperative launch against a
 * regular one.  They are measurement, not part of the exchange: they give
 * the achievable ceiling against which the exchange's bandwidth is read,
 * beside the published HBM peak, and the fixed cost its final launch pays
 * when it is cooperative.
 *
 * Each probe streams `bytes` through the same instructions and launch shape
 * as the segment-copy kernel's byte copy: 1024-thread workgroups (one per
 * compute unit unless `workgroups` says otherwise), 64 KiB tiles claimed from
 * a counter in tile order, 16-byte streaming loads (buffer_load nt) with 4
 * words in flight per lane, 16-byte streaming device-scope stores
 * (buffer_store nt sc1).
 *   A2AV_PROBE_READ   reads src; writes nothing (dst may be NULL)
 *   A2AV_PROBE_WRITE  writes the 32-bit pattern 0xA5A5A5A5 into dst; reads nothing
 *   A2AV_PROBE_COPY   copies src to dst
 * src and dst are device pointers, 16-byte aligned; `bytes` is a positive
 * multiple of 16 below 2^40.  The call enqueues one launch on `stream` and
 * does not synchronize.  Calls that overlap on one device share the tile
 * counter and race: order them.
 * Returns A2AV_OK, A2AV_ERR_NULLPTR, A2AV_ERR_INVALID_ARGS (kind, size,
 * alignment, workgroups < 0) or A2AV_ERR_HIP (a2av.h's status values).
 */
#ifndef A2AV_PROBE_H
#define A2AV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum a2av_probe_kind { A2AV_PROBE_READ = 0, A2AV_PROBE_WRITE = 1, A2AV_PROBE_COPY = 2 };

int a2av_probe_stream(int32_t kind, const void *src, void *dst, int64_t bytes,
                      int32_t workgroups, void *stream);

/*
 * Launch probe: one launch of `workgroups` 1024-thread workgroups (0 = one
 * per compute unit) that stores `bytes` bytes of the pattern 0xA5 into dst
 * with the copy kernel's store instruction (buffer_store nt sc1, grid-stride;
 * bytes = 0 stores nothing), enqueued on `stream` either as a regular launch
 * (cooperative = 0, hipLaunchKernel) or as a cooperative one (cooperative =
 * 1, hipLaunchCooperativeKernel, as the exchange's final launch when it
 * admits more than one block).  Timing launches of each kind back to back
 * gives the cooperative launch's own cost on the stream, apart from any
 * exchange.  Measurement only.  dst is a device pointer, 16-byte aligned,
 * and may be NULL when bytes = 0; bytes is a multiple of 16 in [0, 2^31).
 * The call does not synchronize.
 * Returns A2AV_OK, A2AV_ERR_NULLPTR, A2AV_ERR_INVALID_ARGS (cooperative not
 * 0 or 1, size, alignment, workgroups < 0), A2AV_ERR_LAUNCH_CAPACITY (a
 * cooperative grid the device cannot hold at once) or A2AV_ERR_HIP.
 */
int a2av_probe_launch(int32_t cooperative, void *dst, int64_t bytes, int32_t workgroups,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* A2AV_PROBE_H */
