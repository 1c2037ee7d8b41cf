// plan.cpp -- host-side planning (see plan.h).  No HIP calls: these functions
// are exported through the C ABI and tested on machines without a GPU.
#include "plan.h"

#include <algorithm>

namespace a2av {

int64_t fold_blocks(int64_t P, int64_t L) {
  if (P < 1 || L < 1) return -1;
  return L < P ? L : (L / P) * P;
}

int64_t elem_bytes(int32_t dtype) {
  return dtype == A2AV_FP32 ? 4 : dtype == A2AV_INT8 ? 1 : 2;
}

int check_config(const a2av_config* cfg) {
  if (!cfg) return A2AV_ERR_NULLPTR;
  if (cfg->P < 1 || cfg->P > kMaxP) return A2AV_ERR_INVALID_ARGS;
  if (cfg->in_slab_bytes < 1 || cfg->tgt_slab_bytes < 1) return A2AV_ERR_INVALID_ARGS;
  if (cfg->S < 1) return A2AV_ERR_INVALID_ARGS;
  if (cfg->chunk_limit_bytes < 0 || cfg->capacity_override < 0) return A2AV_ERR_INVALID_ARGS;
  if (cfg->wg_per_block < 0 || cfg->spin_limit < 0) return A2AV_ERR_INVALID_ARGS;
  // Slab offsets are formed in 64-bit arithmetic; keep P * slab far from overflow.
  if (cfg->in_slab_bytes > (int64_t(1) << 46) || cfg->tgt_slab_bytes > (int64_t(1) << 46))
    return A2AV_ERR_INVALID_ARGS;
  // A chunk limit so small that the payload bound needs more than
  // kMaxLaunches launches is refused.
  const int64_t limit = cfg->chunk_limit_bytes > 0 ? cfg->chunk_limit_bytes : kDefaultChunkLimit;
  if ((max_payload(cfg) + limit - 1) / limit > kMaxLaunches) return A2AV_ERR_INVALID_ARGS;
  return A2AV_OK;
}

namespace {

struct Range {
  uintptr_t lo;
  uint64_t len;
};

bool overlap(const Range& a, const Range& b) {
  if (a.len == 0 || b.len == 0) return false;
  return a.lo < b.lo + b.len && b.lo < a.lo + a.len;
}

}  // namespace

int check_run_args(const a2av_config* cfg, int64_t capacity, const void* input,
                   const void* target, const int32_t* signal, const int32_t* send_counts,
                   const int32_t* recv_counts, int32_t P, int64_t core_num, int32_t dtype,
                   int32_t nblk) {
  if (!cfg || !input || !target || !signal || !send_counts || !recv_counts)
    return A2AV_ERR_NULLPTR;
  if (dtype != A2AV_FP32 && dtype != A2AV_INT8) return A2AV_ERR_UNSUPPORTED_DTYPE;
  if (check_config(cfg) != A2AV_OK) return A2AV_ERR_INVALID_ARGS;
  if (P != cfg->P || nblk < 1) return A2AV_ERR_INVALID_ARGS;
  if (core_num < 1 || core_num > kInt32Max) return A2AV_ERR_INVALID_ARGS;
  const int64_t B = fold_blocks(P, core_num);
  if (int64_t(cfg->S) < B) return A2AV_ERR_INVALID_ARGS;
  if (B > 1 && capacity > 0 && B > capacity) return A2AV_ERR_LAUNCH_CAPACITY;

  const uint64_t p = uint64_t(P);
  const Range r[5] = {
      {uintptr_t(input), p * uint64_t(cfg->in_slab_bytes)},
      {uintptr_t(target), p * uint64_t(cfg->tgt_slab_bytes)},
      {uintptr_t(signal), p * uint64_t(cfg->S) * 4u},
      {uintptr_t(send_counts), p * p * 4u},
      {uintptr_t(recv_counts), p * p * 4u},
  };
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(r[i], r[j])) return A2AV_ERR_INVALID_ARGS;

  const int64_t e = elem_bytes(dtype);
  if (cfg->in_slab_bytes % e != 0 || cfg->tgt_slab_bytes % e != 0) return A2AV_ERR_INVALID_ARGS;
  return A2AV_OK;
}

int check_bias_args(const a2av_config* cfg, int64_t capacity, int64_t chunk_limit,
                    const void* input, const void* target, const int32_t* signal,
                    const int32_t* send_counts, const int32_t* recv_counts, const void* bias,
                    int32_t P, int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden) {
  if (!cfg || !input || !target || !signal || !send_counts || !recv_counts || !bias)
    return A2AV_ERR_NULLPTR;
  if (dtype != A2AV_FP16 && dtype != A2AV_BF16) return A2AV_ERR_UNSUPPORTED_DTYPE;
  if (check_config(cfg) != A2AV_OK) return A2AV_ERR_INVALID_ARGS;
  if (P != cfg->P || nblk < 1 || hidden < 1) return A2AV_ERR_INVALID_ARGS;
  if (core_num < 1 || core_num > kInt32Max) return A2AV_ERR_INVALID_ARGS;
  const int64_t B = fold_blocks(P, core_num);
  if (int64_t(cfg->S) < B) return A2AV_ERR_INVALID_ARGS;
  if (B > 1 && capacity > 0 && B > capacity) return A2AV_ERR_LAUNCH_CAPACITY;

  const uint64_t p = uint64_t(P);
  const uint64_t bias_e = dtype == A2AV_BF16 ? 4u : 2u;
  const Range r[6] = {
      {uintptr_t(input), p * uint64_t(cfg->in_slab_bytes)},
      {uintptr_t(target), p * uint64_t(cfg->tgt_slab_bytes)},
      {uintptr_t(signal), p * uint64_t(cfg->S) * 4u},
      {uintptr_t(send_counts), p * p * 4u},
      {uintptr_t(recv_counts), p * p * 4u},
      {uintptr_t(bias), p * uint64_t(nblk) * uint64_t(hidden) * bias_e},
  };
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlap(r[i], r[j])) return A2AV_ERR_INVALID_ARGS;
  if (cfg->in_slab_bytes % 2 != 0 || cfg->tgt_slab_bytes % 2 != 0) return A2AV_ERR_INVALID_ARGS;
  // Limits of the GPU path: 16-byte rows and 16-byte aligned operands, so
  // every piece is whole 16-byte words of one row.
  if (hidden % 8 != 0 || hidden > kMaxHidden) return A2AV_ERR_INVALID_ARGS;
  if (((uintptr_t(input) | uintptr_t(target) | uintptr_t(bias)) & 15u) != 0)
    return A2AV_ERR_INVALID_ARGS;
  if (cfg->in_slab_bytes % 16 != 0 || cfg->tgt_slab_bytes % 16 != 0 || chunk_limit % 16 != 0)
    return A2AV_ERR_INVALID_ARGS;
  return A2AV_OK;
}

int check_indexed_args(const a2av_config* cfg, int64_t capacity, const void* input,
                       const void* target, const int32_t* signal, const int32_t* send_counts,
                       const int32_t* recv_counts, const int32_t* index, int32_t P,
                       int64_t core_num, int32_t dtype, int32_t row_elems, int64_t index_stride) {
  if (!cfg || !input || !target || !signal || !send_counts || !recv_counts || !index)
    return A2AV_ERR_NULLPTR;
  if (dtype != A2AV_FP32 && dtype != A2AV_INT8) return A2AV_ERR_UNSUPPORTED_DTYPE;
  if (check_config(cfg) != A2AV_OK) return A2AV_ERR_INVALID_ARGS;
  if (P != cfg->P || row_elems < 1 || index_stride < 1) return A2AV_ERR_INVALID_ARGS;
  // Keep P * index_stride entries far from 64-bit overflow.
  if (index_stride > (int64_t(1) << 40)) return A2AV_ERR_INVALID_ARGS;
  // A chunk limit that needs more than kMaxLaunches launches to cover the
  // largest gathered payload is refused.
  const int64_t limit = cfg->chunk_limit_bytes > 0 ? cfg->chunk_limit_bytes : kDefaultChunkLimit;
  const int64_t row_bytes = int64_t(row_elems) * elem_bytes(dtype);
  const int64_t bound = gather_max_payload(cfg, row_bytes, index_stride);
  if ((bound + limit - 1) / limit > kMaxLaunches) return A2AV_ERR_INVALID_ARGS;
  if (core_num < 1 || core_num > kInt32Max) return A2AV_ERR_INVALID_ARGS;
  const int64_t B = fold_blocks(P, core_num);
  if (int64_t(cfg->S) < B) return A2AV_ERR_INVALID_ARGS;
  if (B > 1 && capacity > 0 && B > capacity) return A2AV_ERR_LAUNCH_CAPACITY;

  const uint64_t p = uint64_t(P);
  const Range r[6] = {
      {uintptr_t(input), p * uint64_t(cfg->in_slab_bytes)},
      {uintptr_t(target), p * uint64_t(cfg->tgt_slab_bytes)},
      {uintptr_t(signal), p * uint64_t(cfg->S) * 4u},
      {uintptr_t(send_counts), p * p * 4u},
      {uintptr_t(recv_counts), p * p * 4u},
      {uintptr_t(index), p * uint64_t(index_stride) * 4u},
  };
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlap(r[i], r[j])) return A2AV_ERR_INVALID_ARGS;
  const int64_t e = elem_bytes(dtype);
  if (cfg->in_slab_bytes % e != 0 || cfg->tgt_slab_bytes % e != 0) return A2AV_ERR_INVALID_ARGS;
  return A2AV_OK;
}

int64_t max_payload(const a2av_config* cfg) {
  return int64_t(cfg->P) * std::min(cfg->in_slab_bytes, cfg->tgt_slab_bytes);
}

int64_t gather_max_payload(const a2av_config* cfg, int64_t row_bytes, int64_t index_stride) {
  const int64_t by_target = int64_t(cfg->P) * cfg->tgt_slab_bytes;
  // index_stride <= by_target / row_bytes / P keeps the product below
  // by_target, so it cannot overflow.
  if (row_bytes < 1 || index_stride > by_target / row_bytes / cfg->P) return by_target;
  return int64_t(cfg->P) * index_stride * row_bytes;
}

int32_t chunk_launches(const a2av_config* cfg, int64_t limit) {
  const int64_t t = max_payload(cfg);
  const int64_t n = (t + limit - 1) / limit;
  return int32_t(std::max<int64_t>(1, n));
}

int check_host_counts(const a2av_config* cfg, const int32_t* counts, int64_t elem,
                      int64_t unit, int64_t index_stride, int64_t* payload) {
  const int32_t P = cfg->P;
  const int64_t PP = int64_t(P) * P;
  for (int64_t i = 0; i < PP; ++i)
    if (counts[i] < 0) return A2AV_ERR_INVALID_ARGS;
  for (int64_t i = 0; i < PP; ++i)
    if (counts[i] % unit != 0) return A2AV_ERR_INVALID_ARGS;
  int64_t total = 0;
  for (int32_t s = 0; s < P; ++s) {
    int64_t row = 0;
    for (int32_t d = 0; d < P; ++d) row += counts[int64_t(s) * P + d];
    if (index_stride > 0 ? row / unit > index_stride : row * elem > cfg->in_slab_bytes)
      return A2AV_ERR_OVER_CAPACITY;
    total += row * elem;
  }
  for (int32_t d = 0; d < P; ++d) {
    int64_t col = 0;
    for (int32_t s = 0; s < P; ++s) col += counts[int64_t(s) * P + d];
    if (col * elem > cfg->tgt_slab_bytes) return A2AV_ERR_OVER_CAPACITY;
  }
  *payload = total;
  return A2AV_OK;
}

int32_t launches_for(int64_t payload, int64_t limit) {
  return int32_t(std::max<int64_t>(1, (payload + limit - 1) / limit));
}

int32_t wg_per_block(int64_t B, int64_t capacity, int64_t payload_bound, int32_t requested,
                     int64_t target_wgs, int64_t min_bytes_per_wg) {
  if (B < 1) return 1;
  const int64_t cap_g = capacity > 0 ? std::max<int64_t>(1, capacity / B) : int64_t(1) << 20;
  if (requested > 0) return int32_t(std::min<int64_t>(requested, cap_g));
  int64_t g = (target_wgs + B - 1) / B;
  const int64_t by_bytes = payload_bound / (B * std::max<int64_t>(1, min_bytes_per_wg));
  g = std::min(g, std::max<int64_t>(1, by_bytes));
  g = std::min(g, cap_g);
  return int32_t(std::max<int64_t>(1, g));
}

}  // namespace a2av
