// probe.hip -- the probes of include/a2av_probe.h: read-only, write-only and
// copy kernels built from the copy kernel's memory instructions and launch
// shape, to measure the rates those instructions reach on the device (the
// exchange's achievable ceiling); and a store kernel launched either as a
// regular or as a cooperative launch, to measure what the cooperative launch
// itself costs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "a2av.h"
#include "a2av_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 1024;       // as the copy kernel's workgroups
constexpr int kUnroll = 4;           // 16-byte words in flight per lane
constexpr int64_t kTile = 65536;     // bytes per claimed tile (one pass)
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadPolicy = 2;       // nt
constexpr int kStorePolicy = 2 | 16; // nt sc1

// Tile claims of the running probe, and its workgroups done with them: the
// last workgroup out clears both, so every launch starts from zero.
__device__ uint32_t g_claim;
__device__ uint32_t g_exited;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(n), kRsrcWord3);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void probe_kernel(const uint8_t* src, uint8_t* dst,
                                                         int64_t bytes, int32_t never) {
  __shared__ int64_t s_tile;
  const int tid = threadIdx.x;
  const int64_t ntiles = (bytes + kTile - 1) / kTile;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  const u32x4 pattern = u32x4{0xA5A5A5A5u, 0xA5A5A5A5u, 0xA5A5A5A5u, 0xA5A5A5A5u};
  if (tid == 0)
    s_tile = int64_t(__hip_atomic_fetch_add(&g_claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  __syncthreads();
  int64_t t = s_tile;
  while (t < ntiles) {
    uint32_t next = 0u;
    if (tid == 0)
      next = __hip_atomic_fetch_add(&g_claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t lo = t * kTile;
    const int64_t n = bytes - lo < kTile ? bytes - lo : kTile;
    const int64_t K = n >> 4;
    const __amdgpu_buffer_rsrc_t rs = rsrc(src + (KIND == A2AV_PROBE_WRITE ? 0 : lo), n);
    const __amdgpu_buffer_rsrc_t rd = rsrc(dst + (KIND == A2AV_PROBE_READ ? 0 : lo), n);
    for (int64_t k0 = 0; k0 < K; k0 += int64_t(kThreads) * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t k = k0 + int64_t(j) * kThreads + tid;
        v[j] = pattern;
        if (KIND != A2AV_PROBE_WRITE && k < K)
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, int(k * 16), 0, kLoadPolicy);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t k = k0 + int64_t(j) * kThreads + tid;
        if (k >= K) continue;
        if (KIND == A2AV_PROBE_READ)
          acc ^= v[j];
        else
          __builtin_amdgcn_raw_buffer_store_b128(v[j], rd, int(k * 16), 0, kStorePolicy);
      }
    }
    __syncthreads();
    if (tid == 0) s_tile = int64_t(next);
    __syncthreads();
    t = s_tile;
  }
  // The read probe keeps its loads alive through a store the host never asks
  // for (never = 0).
  if (KIND == A2AV_PROBE_READ && never)
    reinterpret_cast<u32x4*>(dst)[blockIdx.x * kThreads + tid] = acc;
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(&g_exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1u) {
      __hip_atomic_store(&g_claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&g_exited, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The launch probe: each thread stores its 16-byte words of `bytes` with the
// copy kernel's store instruction, grid-stride; bytes = 0 stores nothing.
__global__ __launch_bounds__(kThreads) void launch_probe_kernel(uint8_t* dst, int64_t bytes) {
  const int64_t K = bytes >> 4;
  if (K == 0) return;
  const __amdgpu_buffer_rsrc_t rd = rsrc(dst, bytes);
  const u32x4 pattern = u32x4{0xA5A5A5A5u, 0xA5A5A5A5u, 0xA5A5A5A5u, 0xA5A5A5A5u};
  for (int64_t k = int64_t(blockIdx.x) * kThreads + threadIdx.x; k < K;
       k += int64_t(gridDim.x) * kThreads)
    __builtin_amdgcn_raw_buffer_store_b128(pattern, rd, int(k * 16), 0, kStorePolicy);
}

}  // namespace

extern "C" int a2av_probe_launch(int32_t cooperative, void* dst, int64_t bytes,
                                 int32_t workgroups, void* stream) {
  if (cooperative != 0 && cooperative != 1) return A2AV_ERR_INVALID_ARGS;
  if (bytes < 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 31) || workgroups < 0)
    return A2AV_ERR_INVALID_ARGS;
  if (bytes > 0 && !dst) return A2AV_ERR_NULLPTR;
  if ((uintptr_t(dst) & 15u) != 0) return A2AV_ERR_INVALID_ARGS;
  int W = workgroups;
  if (W == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&W, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return A2AV_ERR_HIP;
    }
  }
  uint8_t* d = static_cast<uint8_t*>(dst);
  void* args[] = {&d, &bytes};
  const void* f = reinterpret_cast<const void*>(&launch_probe_kernel);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = cooperative
                           ? hipLaunchCooperativeKernel(f, dim3(W), dim3(kThreads), args, 0, s)
                           : hipLaunchKernel(f, dim3(W), dim3(kThreads), args, 0, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return cooperative && e == hipErrorCooperativeLaunchTooLarge ? A2AV_ERR_LAUNCH_CAPACITY
                                                                 : A2AV_ERR_HIP;
  }
  return A2AV_OK;
}

extern "C" int a2av_probe_stream(int32_t kind, const void* src, void* dst, int64_t bytes,
                                 int32_t workgroups, void* stream) {
  if (kind != A2AV_PROBE_READ && kind != A2AV_PROBE_WRITE && kind != A2AV_PROBE_COPY)
    return A2AV_ERR_INVALID_ARGS;
  if ((kind != A2AV_PROBE_WRITE && !src) || (kind != A2AV_PROBE_READ && !dst))
    return A2AV_ERR_NULLPTR;
  if (bytes < 16 || bytes % 16 != 0 || bytes >= (int64_t(1) << 40) || workgroups < 0)
    return A2AV_ERR_INVALID_ARGS;
  if (((uintptr_t(src) | uintptr_t(dst)) & 15u) != 0) return A2AV_ERR_INVALID_ARGS;
  int W = workgroups;
  if (W == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&W, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return A2AV_ERR_HIP;
    }
  }
  const void* f = kind == A2AV_PROBE_READ    ? reinterpret_cast<const void*>(&probe_kernel<0>)
                  : kind == A2AV_PROBE_WRITE ? reinterpret_cast<const void*>(&probe_kernel<1>)
                                             : reinterpret_cast<const void*>(&probe_kernel<2>);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  int32_t never = 0;
  void* args[] = {&s, &d, &bytes, &never};
  if (hipLaunchKernel(f, dim3(W), dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) !=
      hipSuccess) {
    (void)hipGetLastError();
    return A2AV_ERR_HIP;
  }
  return A2AV_OK;
}
