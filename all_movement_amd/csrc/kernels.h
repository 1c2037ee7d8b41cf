// kernels.h -- device-side data shared by the count kernel (K1) and the
// segment-copy kernel (K2), and their launch parameters.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace a2av {

// Words written by K1 for one run and read by every K2 launch of that run.
struct alignas(64) RunPlan {
  int32_t valid;        // 1 when the run's counts and signal passed the device checks
  int32_t error;        // latched status (first failure since the last query)
  int64_t total_bytes;  // payload bytes T of the run
  uint64_t kstate;      // K1's verdict word (0 between runs): 8-bit fields, the
                        // workgroups done in the lowest, then per failure kind
                        // the workgroups that found it
  uint32_t claim[2];    // dynamic tile counters; K2 launch c uses claim[c & 1]
};

// The arrival counter of the final launch is kept in kArriveReplicas copies,
// kArriveStride words (256 bytes) apart: every arriving block adds 1 to each
// copy (one lane per copy) and workgroup w polls copy w % kArriveReplicas.
// With a single counter the polls of the waiting workgroups all landed on one
// memory channel and slowed the copies still running (gfx950, c4's 256-block
// launch: 324 -> 308 us).
constexpr int kArriveReplicas = 64;
constexpr int kArriveStride = 64;

// Device workspace layout, carved out of one allocation by the host.
struct Workspace {
  RunPlan* plan;
  int64_t* prefix;   // [nseg + 1] exclusive prefix of segment bytes in the flattened
                     // order (d-major, or s-major for the row gather); nseg = P*P, or
                     // P*P*nblk when the blocked byte copy takes a segment per sub-block
  int64_t* src_off;  // [nseg] byte offset inside `input` of each segment, flattened order
  int64_t* dst_off;  // [nseg] byte offset inside `target` of each segment, flattened order
  uint32_t* blk_cnt; // [max blocks] workgroups of each block that finished copying
  int64_t* sstride;  // [P] bytes per source block-row (blocked exchange)
  uint32_t* arrived; // [kArriveReplicas * kArriveStride] admitted blocks that have raised
                     // their flags, copy k at arrived[k * kArriveStride]
};

struct CountParams {
  const int32_t* send_counts;
  const int32_t* signal;
  Workspace ws;
  int64_t in_slab;
  int64_t tgt_slab;
  int32_t P;
  int32_t S;
  int32_t B;
  int32_t elem;
  int32_t nblk;       // sub-blocks per segment (1 = plain exchange)
  int32_t expand;     // 1: one table entry per sub-block (P * P * nblk entries, byte copy)
  int64_t unit;       // every count must be a multiple of this (nblk, nblk * hidden, or a row)
  // Indexed exchange only (index != nullptr): the gather lists, their
  // stride, and the whole rows each input table holds.
  const int32_t* index;
  int64_t index_stride;
  int64_t table_rows;
  int64_t payload_cap;  // bytes the run's launches cover; a larger payload is refused
  int32_t* status_out;  // if set: receives the run's device-side status (0 = valid)
};

struct CopyParams {
  const uint8_t* input;
  uint8_t* target;
  int32_t* signal;
  const int32_t* send_counts;
  int32_t* recv_counts;  // written by the final launch, once the run's checks passed
  Workspace ws;
  int64_t chunk_lo;   // flattened payload range of this launch (clamped to T on device)
  int64_t chunk_hi;
  int32_t nseg;       // P*P
  int32_t P;
  int32_t S;
  int32_t B;
  int32_t G;          // workgroups per admitted block
  int32_t nblk;       // sub-blocks per segment (1 = plain exchange)
  int32_t mode;       // 0: move bytes; 1: BF16 + FP32 bias; 2: FP16 + FP16 bias; 3: row gather
  int32_t hidden;     // elements per row (bias modes)
  const void* bias;   // [P, nblk, hidden] (bias modes)
  const int32_t* index;   // gather lists [P, index_stride] (mode 3)
  int64_t index_stride;
  int64_t in_slab;
  int64_t row_bytes;      // bytes per gathered row (mode 3)
  int32_t gather_words;   // mode 3: 1 when every row and operand is 16-byte aligned
  int32_t chunk;      // chunk index of this launch (launches run from the highest to 0)
  int32_t last;       // 1 on the run's final launch: raise the block flags
  int32_t wait;       // 1 when the final launch is cooperative (B > 1): wait for all blocks
  int32_t spin_limit;
  int32_t* status_out;  // if set: receives TIMEOUT when the block barrier times out
};

constexpr int kCountThreads = 1024;
constexpr int kCopyThreads = 1024;  // K2 workgroups of the plain, blocked and indexed exchanges
// K2 workgroups of the fused-bias exchange: 512 threads with 8 words in flight
// per lane, 64 KiB tiles (measured on gfx950 against 1024 threads and 128 KiB
// tiles: c5b 6,114 -> 6,324 GB/s over the whole run, c5h 6,247 -> 6,455).
constexpr int kBiasThreads = 512;

// Launch helpers (defined in kernels.hip).
hipError_t launch_count(const CountParams& p, int workgroups, hipStream_t stream);
hipError_t launch_copy(const CopyParams& p, int workgroups, bool cooperative, hipStream_t stream);
hipError_t copy_occupancy(int* wgs_per_cu);

}  // namespace a2av
