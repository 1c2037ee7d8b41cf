// plan.h -- host-side planning for the all_to_all_v library: the block fold,
// the argument checks that run before anything is enqueued, the chunk plan
// and the workgroups-per-block choice.  Pure C++ (no HIP calls).
#pragma once

#include <cstdint>

#include "a2av.h"

namespace a2av {

constexpr int32_t kMaxP = 64;
constexpr int64_t kDefaultChunkLimit = int64_t(1) << 30;
// At most this many K2 launches per run (the chunk plan's launch count is an
// int32 and every launch costs microseconds; 2^20 GiB-sized chunks is far
// beyond any device's memory).
constexpr int64_t kMaxLaunches = int64_t(1) << 20;
constexpr int64_t kInt32Max = 2147483647LL;
// Longest bias row of a2av_run_bias: the row's bytes must stay a 32-bit
// buffer offset.
constexpr int32_t kMaxHidden = int32_t(1) << 28;

// CalAllToAllVBlocks(P, L) ("Launch width" section of the PyPTO
// LowerL2TensorCollectives page): L below P stays L, otherwise the largest
// multiple of P that does not exceed L.  -1 on P < 1 or L < 1.
int64_t fold_blocks(int64_t P, int64_t L);

int64_t elem_bytes(int32_t dtype);

// Geometry checks done once by a2av_create.
int check_config(const a2av_config* cfg);

// The host-side checks of a2av_run / a2av_run_blocked, in the documented
// order (nblk = 1 for a2av_run).
int check_run_args(const a2av_config* cfg, int64_t capacity, const void* input,
                   const void* target, const int32_t* signal, const int32_t* send_counts,
                   const int32_t* recv_counts, int32_t P, int64_t core_num, int32_t dtype,
                   int32_t nblk = 1);

// The host-side checks of a2av_run_bias (fused bias Add, 16-bit payloads),
// in the documented order; chunk_limit is the handle's bytes per launch.
int check_bias_args(const a2av_config* cfg, int64_t capacity, int64_t chunk_limit,
                    const void* input, const void* target, const int32_t* signal,
                    const int32_t* send_counts, const int32_t* recv_counts, const void* bias,
                    int32_t P, int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden);

// The host-side checks of a2av_run_indexed, in the documented order.
int check_indexed_args(const a2av_config* cfg, int64_t capacity, const void* input,
                       const void* target, const int32_t* signal, const int32_t* send_counts,
                       const int32_t* recv_counts, const int32_t* index, int32_t P,
                       int64_t core_num, int32_t dtype, int32_t row_elems, int64_t index_stride);

// Upper bound of the payload of any valid run.  Every destination column
// fits its target slab, so T <= P * tgt_slab always; in the exchanges that
// read each input byte at most once every source row also fits its input
// slab, so T <= P * min(in_slab, tgt_slab).
int64_t max_payload(const a2av_config* cfg);

// The same bound for the row gather, which may name a row any number of
// times: the target bound, and every source sending at most index_stride
// rows of row_bytes bytes (its gather list), whichever is smaller.
int64_t gather_max_payload(const a2av_config* cfg, int64_t row_bytes, int64_t index_stride);

// K2 launches per run: enough chunks of `limit` bytes to cover max_payload.
// Launch c copies the flattened payload bytes [c * limit, (c + 1) * limit);
// the device skips the part of a chunk past the run's real payload.
int32_t chunk_launches(const a2av_config* cfg, int64_t limit);

// The device's count checks on a host copy of the counts (elements of
// `elem` bytes), in the device's order: a negative count (INVALID_ARGS); a
// count that `unit` does not divide (INVALID_ARGS: not whole sub-blocks, bias
// rows or gathered rows; unit 1 for the plain exchange); a source row over
// its limit (over in_slab bytes, or with index_stride > 0 more than
// index_stride rows of `unit` elements) or a destination column over
// tgt_slab (OVER_CAPACITY).  On success *payload is the run's payload in
// bytes.
int check_host_counts(const a2av_config* cfg, const int32_t* counts, int64_t elem,
                      int64_t unit, int64_t index_stride, int64_t* payload);

// Launches of at most `limit` bytes that cover `payload` (at least one: the
// final launch also writes recv_counts and raises the flags).
int32_t launches_for(int64_t payload, int64_t limit);

// Workgroups that execute one admitted block.  `requested` > 0 is taken as
// is (clamped to the capacity); 0 picks enough to cover `target_wgs`
// workgroups without giving any workgroup less than `min_bytes_per_wg` of the
// payload bound, and never more than capacity / B.
int32_t wg_per_block(int64_t B, int64_t capacity, int64_t payload_bound, int32_t requested,
                     int64_t target_wgs, int64_t min_bytes_per_wg);

}  // namespace a2av
