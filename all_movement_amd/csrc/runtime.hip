// runtime.hip -- the C ABI of include/a2av.h: handle lifetime, host checks,
// the chunk plan, and the K1 + K2 launch sequence of one exchange.
//
// One run enqueues, on the caller's stream and without synchronizing:
//   K1  count_kernel            (1 workgroup)       device checks, segment offsets,
//                                                   payload prefix (workspace only)
//   K2  copy_kernel x launches  (B*G workgroups)    launch c copies payload bytes
//                                                   [c*limit, (c+1)*limit) of the
//                                                   flattened payload order
// The number of K2 launches comes from the slab geometry (the payload bound
// P * min(in_slab, tgt_slab)), so the host never reads the counts back; a
// launch whose range lies past the run's payload does no copying.  Launches
// go from the highest chunk down to chunk 0; only the final one (chunk 0)
// writes recv_counts and raises the signal flags, and it is cooperative when
// B > 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "a2av.h"
#include "kernels.h"
#include "plan.h"

struct a2av_handle {
  a2av_config cfg{};
  int device = 0;
  int cus = 0;
  int wgs_per_cu = 0;
  int64_t capacity = 0;      // co-resident copy workgroups
  int64_t chunk_limit = 0;
  int32_t launches = 1;
  int32_t spin_limit = 0;
  void* ws_mem = nullptr;
  a2av::Workspace ws{};
  hipStream_t last_stream = nullptr;
  bool profile = false;
  // Event sets of the last kProfileRuns runs: per run [0] before K1, [1] after
  // K1, [2] after the last K2 launch (one marker per K2 launch cost c5 ~1 %).
  std::vector<hipEvent_t> events;
  std::vector<int32_t> run_launches;  // K2 launches of each recorded run
  int32_t events_per_run = 0;
  int64_t profiled_runs = 0;  // runs recorded since the last a2av_profile_read
  int64_t run_counter = 0;    // runs recorded
  int32_t profile_every = 1;  // record one run in profile_every ...
  int64_t enqueued = 0;       // ... counting the runs enqueued since it was set
  std::string last_error;
  // Runs of a2av_run_noalloc: the device word that receives each run's
  // device-side status, and no stored error text (storing it allocates).
  int32_t* status_out = nullptr;
  bool keep_error_text = true;
};

namespace {

// Auto G aims at one workgroup per CU, but gives no workgroup less than
// kMinBytesPerWg of the payload bound.  Small exchanges are latency-bound, and
// more workgroups shorten them: c2 (P = 8, 1 MiB bound, B = 8) measured 39.9 /
// 36.8 / 35.4 / 34.3 / 34.3 us per run with 256 / 64 / 32 / 16 / 8 KiB (8 to
// 128 workgroups), and 20.4 -> 14.9 us at 16 KiB without the block wait.  The
// large workloads reach one workgroup per CU either way.
constexpr int64_t kTargetWgsPerCu = 1;
constexpr int64_t kMinBytesPerWg = 16 * 1024;
constexpr int32_t kDefaultSpinLimit = 1 << 22;
constexpr int64_t kProfileRuns = 256;           // runs whose event sets are kept

class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
    if (prev_ != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
  }

 private:
  int prev_ = -1;
};

int hip_fail(a2av_handle* h, hipError_t e, const char* what) {
  if (h && h->keep_error_text) {
    h->last_error = std::string(what) + ": " + hipGetErrorString(e);
  }
  // The status carries the failure: clear HIP's per-thread last error so a
  // later, unrelated call does not report it again.
  (void)hipGetLastError();
  return A2AV_ERR_HIP;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Segment table entries a handle's workspace holds (the most K2's LDS tables
// take): room for one segment per sub-block of the blocked byte copy when
// P * P * nblk fits.
constexpr size_t kMaxSegs = size_t(a2av::kMaxP) * a2av::kMaxP;

// The workspace of a run for P ranks and up to `capacity` admitted blocks:
// plan words, prefix[E+1], src_off[E], dst_off[E] (E = the larger of P*P
// and table_entries), blk_cnt[max(1, capacity)], sstride[P], the arrival
// counter copies, each 256-byte aligned.  Returns its size in bytes; with a
// base address, also fills *ws.
size_t carve_workspace(char* base, int32_t P, int64_t capacity, a2av::Workspace* ws,
                       size_t table_entries) {
  const size_t PP = std::max(size_t(P) * size_t(P), table_entries);
  const size_t max_blocks = size_t(capacity > 1 ? capacity : 1);
  size_t off = 0;
  const size_t o_plan = off; off = round_up(off + sizeof(a2av::RunPlan), 256);
  const size_t o_prefix = off; off = round_up(off + (PP + 1) * sizeof(int64_t), 256);
  const size_t o_src = off; off = round_up(off + PP * sizeof(int64_t), 256);
  const size_t o_dst = off; off = round_up(off + PP * sizeof(int64_t), 256);
  const size_t o_cnt = off; off = round_up(off + max_blocks * sizeof(uint32_t), 256);
  const size_t o_str = off; off = round_up(off + size_t(P) * sizeof(int64_t), 256);
  const size_t o_arr = off;
  off = round_up(off + size_t(a2av::kArriveReplicas) * a2av::kArriveStride * sizeof(uint32_t), 256);
  if (base && ws) {
    ws->plan = reinterpret_cast<a2av::RunPlan*>(base + o_plan);
    ws->prefix = reinterpret_cast<int64_t*>(base + o_prefix);
    ws->src_off = reinterpret_cast<int64_t*>(base + o_src);
    ws->dst_off = reinterpret_cast<int64_t*>(base + o_dst);
    ws->blk_cnt = reinterpret_cast<uint32_t*>(base + o_cnt);
    ws->sstride = reinterpret_cast<int64_t*>(base + o_str);
    ws->arrived = reinterpret_cast<uint32_t*>(base + o_arr);
  }
  return off;
}

}  // namespace

extern "C" {

int64_t a2av_blocks(int64_t P, int64_t L) { return a2av::fold_blocks(P, L); }

const char* a2av_status_string(int status) {
  switch (status) {
    case A2AV_OK: return "A2AV_OK";
    case A2AV_ERR_NULLPTR: return "A2AV_ERR_NULLPTR";
    case A2AV_ERR_INVALID_ARGS: return "A2AV_ERR_INVALID_ARGS";
    case A2AV_ERR_UNSUPPORTED_DTYPE: return "A2AV_ERR_UNSUPPORTED_DTYPE";
    case A2AV_ERR_OVER_CAPACITY: return "A2AV_ERR_OVER_CAPACITY";
    case A2AV_ERR_LAUNCH_CAPACITY: return "A2AV_ERR_LAUNCH_CAPACITY";
    case A2AV_ERR_HIP: return "A2AV_ERR_HIP";
    case A2AV_ERR_TIMEOUT: return "A2AV_ERR_TIMEOUT";
    default: return "A2AV_ERR_UNKNOWN";
  }
}

int a2av_check_args(const a2av_config* cfg, int64_t capacity, const void* input,
                    const void* target, const int32_t* signal, const int32_t* send_counts,
                    const int32_t* recv_counts, int32_t P, int64_t core_num, int32_t dtype) {
  return a2av::check_run_args(cfg, capacity, input, target, signal, send_counts, recv_counts, P,
                              core_num, dtype);
}

int a2av_check_bias_args(const a2av_config* cfg, int64_t capacity, const void* input,
                         const void* target, const int32_t* signal, const int32_t* send_counts,
                         const int32_t* recv_counts, const void* bias, int32_t P,
                         int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden) {
  const int64_t limit = cfg && cfg->chunk_limit_bytes > 0 ? cfg->chunk_limit_bytes
                                                          : a2av::kDefaultChunkLimit;
  return a2av::check_bias_args(cfg, capacity, limit, input, target, signal, send_counts,
                               recv_counts, bias, P, core_num, dtype, nblk, hidden);
}

int a2av_check_indexed_args(const a2av_config* cfg, int64_t capacity, const void* input,
                            const void* target, const int32_t* signal,
                            const int32_t* send_counts, const int32_t* recv_counts,
                            const int32_t* index, int32_t P, int64_t core_num, int32_t dtype,
                            int32_t row_elems, int64_t index_stride) {
  return a2av::check_indexed_args(cfg, capacity, input, target, signal, send_counts, recv_counts,
                                  index, P, core_num, dtype, row_elems, index_stride);
}

int a2av_create(a2av_handle** out, const a2av_config* cfg) {
  if (!out || !cfg) return A2AV_ERR_NULLPTR;
  *out = nullptr;
  const int st = a2av::check_config(cfg);
  if (st != A2AV_OK) return st;

  a2av_handle* h = new (std::nothrow) a2av_handle();
  if (!h) return A2AV_ERR_HIP;
  h->cfg = *cfg;
  h->device = cfg->device;
  DeviceGuard guard(h->device);

  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) { delete h; return A2AV_ERR_HIP; }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, h->device);
  if (e != hipSuccess) { delete h; return A2AV_ERR_HIP; }
  h->cus = prop.multiProcessorCount;
  e = a2av::copy_occupancy(&h->wgs_per_cu);
  if (e != hipSuccess) { delete h; return A2AV_ERR_HIP; }
  h->capacity = cfg->capacity_override > 0 ? cfg->capacity_override
                                           : int64_t(h->wgs_per_cu) * h->cus;
  h->chunk_limit = cfg->chunk_limit_bytes > 0 ? cfg->chunk_limit_bytes : a2av::kDefaultChunkLimit;
  h->launches = a2av::chunk_launches(cfg, h->chunk_limit);
  h->spin_limit = cfg->spin_limit > 0 ? cfg->spin_limit : kDefaultSpinLimit;

  const size_t bytes = carve_workspace(nullptr, cfg->P, h->capacity, nullptr, kMaxSegs);
  e = hipMalloc(&h->ws_mem, bytes);
  if (e != hipSuccess) { delete h; return A2AV_ERR_HIP; }
  e = hipMemset(h->ws_mem, 0, bytes);
  if (e != hipSuccess) { (void)hipFree(h->ws_mem); delete h; return A2AV_ERR_HIP; }
  carve_workspace(static_cast<char*>(h->ws_mem), cfg->P, h->capacity, &h->ws, kMaxSegs);

  h->profile = (cfg->flags & A2AV_FLAG_PROFILE) != 0;
  if (h->profile) {
    h->events_per_run = 3;
    h->events.resize(size_t(h->events_per_run) * kProfileRuns, nullptr);
    h->run_launches.assign(size_t(kProfileRuns), 0);
    for (auto& ev : h->events) {
      e = hipEventCreate(&ev);
      if (e != hipSuccess) { a2av_destroy(h); return A2AV_ERR_HIP; }
    }
  }
  *out = h;
  return A2AV_OK;
}

int a2av_destroy(a2av_handle* h) {
  if (!h) return A2AV_OK;
  DeviceGuard guard(h->device);
  (void)hipDeviceSynchronize();
  for (auto& ev : h->events)
    if (ev) (void)hipEventDestroy(ev);
  if (h->ws_mem) (void)hipFree(h->ws_mem);
  delete h;
  return A2AV_OK;
}

int a2av_launch_info_get(a2av_handle* h, int64_t core_num, a2av_launch_info* out) {
  if (!h || !out) return A2AV_ERR_NULLPTR;
  if (core_num < 1 || core_num > a2av::kInt32Max) return A2AV_ERR_INVALID_ARGS;
  const int64_t B = a2av::fold_blocks(h->cfg.P, core_num);
  if (B > 1 && B > h->capacity) return A2AV_ERR_LAUNCH_CAPACITY;
  const int32_t G = a2av::wg_per_block(B, h->capacity, a2av::max_payload(&h->cfg),
                                       h->cfg.wg_per_block, kTargetWgsPerCu * h->cus,
                                       kMinBytesPerWg);
  std::memset(out, 0, sizeof(*out));
  out->blocks = B;
  out->wg_per_block = G;
  out->workgroups = int32_t(B * G);
  out->threads_per_wg = a2av::kCopyThreads;
  out->chunk_launches = h->launches;
  out->chunk_limit_bytes = h->chunk_limit;
  out->capacity = h->capacity;
  out->cooperative = (B > 1 && (h->cfg.flags & A2AV_FLAG_NO_BLOCK_WAIT) == 0) ? 1 : 0;
  return A2AV_OK;
}

}  // extern "C"

namespace {

// What a run adds to the plain exchange (all defaults: the plain exchange).
struct RunExtras {
  int32_t nblk = 1;                // sub-blocks per segment
  const void* bias = nullptr;      // fused bias Add (modes 1, 2)
  int32_t hidden = 0;
  const int32_t* index = nullptr;  // row gather (mode 3)
  int64_t index_stride = 0;
  int32_t row_elems = 0;
  int32_t mode = 0;
  int32_t launches = 0;            // > 0: the run's chunk plan, from a host copy of the counts
};

// Enqueue one run whose arguments passed the host checks: K1, then the K2
// launches.  mode selects the body of K2 (0: move bytes; 1 and 2: the fused
// bias Add for BF16 and FP16 payloads; 3: the row gather).
int enqueue_run(a2av_handle* h, const void* input, void* target, int32_t* signal,
                const int32_t* send_counts, int32_t* recv_counts, int32_t P, int64_t core_num,
                int32_t dtype, const RunExtras& x, void* stream) {
  const int32_t nblk = x.nblk;
  const int32_t mode = x.mode;
  a2av_launch_info li;
  int st = a2av_launch_info_get(h, core_num, &li);
  if (st != A2AV_OK) return st;
  // The row gather's payload has its own bound (a row may be named many
  // times), so it may need more or fewer launches than the handle's plan for
  // the other exchanges.
  const int64_t row_bytes = int64_t(x.row_elems) * a2av::elem_bytes(dtype);
  const int32_t launches =
      x.launches > 0 ? x.launches
      : mode == 3    ? a2av::launches_for(
                        a2av::gather_max_payload(&h->cfg, row_bytes, x.index_stride), h->chunk_limit)
                     : h->launches;

  DeviceGuard guard(h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  h->last_stream = s;
  hipError_t e;

  a2av::CountParams cp{};
  cp.send_counts = send_counts;
  cp.signal = signal;
  cp.ws = h->ws;
  cp.in_slab = h->cfg.in_slab_bytes;
  cp.tgt_slab = h->cfg.tgt_slab_bytes;
  cp.P = P;
  cp.S = h->cfg.S;
  cp.B = int32_t(li.blocks);
  cp.elem = int32_t(a2av::elem_bytes(dtype));
  cp.nblk = nblk;
  // The blocked byte copy takes one segment per sub-block when the tables
  // hold them: K2 then runs the plain exchange's path, which measured faster
  // than walking the sub-blocks of a segment inside each tile (c5's counts
  // with 8 sub-blocks: 2,738 -> 2,686 us per run).  The no-alloc workspace
  // holds P * P entries only, and runs the plain exchange only.
  const bool expand = mode == 0 && nblk > 1 && h->ws_mem != nullptr &&
                      int64_t(P) * P * nblk <= int64_t(kMaxSegs);
  cp.expand = expand ? 1 : 0;
  const int64_t elem = a2av::elem_bytes(dtype);
  if (mode == 3) {
    cp.unit = x.row_elems;
    cp.index = x.index;
    cp.index_stride = x.index_stride;
    cp.table_rows = h->cfg.in_slab_bytes / (int64_t(x.row_elems) * elem);
  } else {
    cp.unit = int64_t(nblk) * (mode != 0 ? x.hidden : 1);
  }
  // What the launches can cover; a payload beyond it (which the capacity
  // checks already rule out) is refused on the device rather than copied in
  // part.
  cp.status_out = h->status_out;
  cp.payload_cap = h->chunk_limit > INT64_MAX / launches ? INT64_MAX
                                                         : int64_t(launches) * h->chunk_limit;

  // Profiling events are not recorded while the stream is being captured
  // into a graph: the host tally counts enqueued runs, and a graph's replays
  // would not pass through it.
  hipEvent_t* ev = nullptr;
  if (h->profile) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(s, &cs)) != hipSuccess)
      return hip_fail(h, e, "hipStreamIsCapturing");
    if (cs == hipStreamCaptureStatusNone && h->enqueued++ % h->profile_every == 0)
      ev = &h->events[size_t(h->run_counter % kProfileRuns) * size_t(h->events_per_run)];
  }
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(h, e, "hipEventRecord");
  // The row gather's K1 checks every gather-list entry in use: beyond 8,192
  // entries its launch spreads them over up to 63 workgroups besides
  // workgroup 0, which writes the tables, about 8,192 entries each.
  int k1_wgs = 1;
  if (mode == 3) {
    const int64_t entries = int64_t(P) * x.index_stride;
    const int64_t checkers = std::min<int64_t>(63, (entries + 8191) / 8192);
    k1_wgs = checkers > 1 ? int(checkers) + 1 : 1;
  }
  if ((e = a2av::launch_count(cp, k1_wgs, s)) != hipSuccess)
    return hip_fail(h, e, "count_kernel launch");
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(h, e, "hipEventRecord");

  a2av::CopyParams kp{};
  kp.input = static_cast<const uint8_t*>(input);
  kp.target = static_cast<uint8_t*>(target);
  kp.signal = signal;
  kp.send_counts = send_counts;
  kp.recv_counts = recv_counts;
  kp.ws = h->ws;
  kp.nseg = expand ? P * P * nblk : P * P;
  kp.P = P;
  kp.S = h->cfg.S;
  kp.B = int32_t(li.blocks);
  kp.G = li.wg_per_block;
  kp.nblk = expand ? 1 : nblk;
  kp.mode = mode;
  kp.hidden = x.hidden;
  kp.bias = x.bias;
  kp.index = x.index;
  kp.index_stride = x.index_stride;
  kp.in_slab = h->cfg.in_slab_bytes;
  kp.row_bytes = int64_t(x.row_elems) * elem;
  // The word gather needs every row start and every piece bound 16-byte
  // aligned on both sides.
  kp.gather_words = mode == 3 && kp.row_bytes % 16 == 0 && (uintptr_t(input) & 15u) == 0 &&
                    (uintptr_t(target) & 15u) == 0 && h->cfg.in_slab_bytes % 16 == 0 &&
                    h->cfg.tgt_slab_bytes % 16 == 0 && h->chunk_limit % 16 == 0;
  kp.spin_limit = h->spin_limit;
  kp.status_out = h->status_out;
  // Chunks are issued from the highest to chunk 0.  Chunks past the run's
  // payload cost only a plain launch that exits at once, and the final launch
  // (the one that raises the flags, cooperative when B > 1) is chunk 0, which
  // holds payload whenever the run has any.  Launch c copies at most the
  // limit: the flattened bytes [c * limit, (c + 1) * limit).
  for (int32_t n = 0; n < launches; ++n) {
    const int32_t c = launches - 1 - n;
    const bool last = (c == 0);
    kp.chunk_lo = int64_t(c) * h->chunk_limit;
    kp.chunk_hi = int64_t(c + 1) * h->chunk_limit;
    kp.chunk = c;
    kp.last = last ? 1 : 0;
    kp.wait = (last && li.cooperative) ? 1 : 0;
    e = a2av::launch_copy(kp, li.workgroups, kp.wait != 0, s);
    if (e != hipSuccess) return hip_fail(h, e, "copy_kernel launch");
  }
  if (ev) {
    if ((e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    h->run_launches[size_t(h->run_counter % kProfileRuns)] = launches;
    ++h->run_counter;
    ++h->profiled_runs;
  }
  return A2AV_OK;
}

}  // namespace

extern "C" {

int a2av_run_blocked(a2av_handle* h, const void* input, void* target, int32_t* signal,
                     const int32_t* send_counts, int32_t* recv_counts, int32_t P,
                     int64_t core_num, int32_t dtype, int32_t nblk, void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  const int st = a2av::check_run_args(&h->cfg, h->capacity, input, target, signal, send_counts,
                                      recv_counts, P, core_num, dtype, nblk);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.nblk = nblk;
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run_bias(a2av_handle* h, const void* input, void* target, int32_t* signal,
                  const int32_t* send_counts, int32_t* recv_counts, const void* bias, int32_t P,
                  int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden, void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  const int st = a2av::check_bias_args(&h->cfg, h->capacity, h->chunk_limit, input, target,
                                       signal, send_counts, recv_counts, bias, P, core_num, dtype,
                                       nblk, hidden);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.nblk = nblk;
  x.bias = bias;
  x.hidden = hidden;
  x.mode = dtype == A2AV_BF16 ? 1 : 2;
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run_indexed(a2av_handle* h, const void* input, void* target, int32_t* signal,
                     const int32_t* send_counts, int32_t* recv_counts, const int32_t* index,
                     int32_t P, int64_t core_num, int32_t dtype, int32_t row_elems,
                     int64_t index_stride, void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  const int st = a2av::check_indexed_args(&h->cfg, h->capacity, input, target, signal,
                                          send_counts, recv_counts, index, P, core_num, dtype,
                                          row_elems, index_stride);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.index = index;
  x.index_stride = index_stride;
  x.row_elems = row_elems;
  x.mode = 3;
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run(a2av_handle* h, const void* input, void* target, int32_t* signal,
             const int32_t* send_counts, int32_t* recv_counts, int32_t P, int64_t core_num,
             int32_t dtype, void* stream) {
  return a2av_run_blocked(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype,
                          1, stream);
}

int a2av_run_host_counts(a2av_handle* h, const void* input, void* target, int32_t* signal,
                         const int32_t* send_counts, int32_t* recv_counts,
                         const int32_t* host_send_counts, int32_t P, int64_t core_num,
                         int32_t dtype, void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  if (!host_send_counts) return A2AV_ERR_NULLPTR;
  int st = a2av::check_run_args(&h->cfg, h->capacity, input, target, signal, send_counts,
                                recv_counts, P, core_num, dtype);
  if (st != A2AV_OK) return st;
  int64_t payload = 0;
  st = a2av::check_host_counts(&h->cfg, host_send_counts, a2av::elem_bytes(dtype), 1, 0, &payload);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.launches = a2av::launches_for(payload, h->chunk_limit);
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run_blocked_host_counts(a2av_handle* h, const void* input, void* target,
                                 int32_t* signal, const int32_t* send_counts,
                                 int32_t* recv_counts, const int32_t* host_send_counts,
                                 int32_t P, int64_t core_num, int32_t dtype, int32_t nblk,
                                 void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  if (!host_send_counts) return A2AV_ERR_NULLPTR;
  int st = a2av::check_run_args(&h->cfg, h->capacity, input, target, signal, send_counts,
                                recv_counts, P, core_num, dtype, nblk);
  if (st != A2AV_OK) return st;
  int64_t payload = 0;
  st = a2av::check_host_counts(&h->cfg, host_send_counts, a2av::elem_bytes(dtype), nblk, 0,
                               &payload);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.nblk = nblk;
  x.launches = a2av::launches_for(payload, h->chunk_limit);
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run_bias_host_counts(a2av_handle* h, const void* input, void* target, int32_t* signal,
                              const int32_t* send_counts, int32_t* recv_counts,
                              const void* bias, const int32_t* host_send_counts, int32_t P,
                              int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden,
                              void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  if (!host_send_counts) return A2AV_ERR_NULLPTR;
  int st = a2av::check_bias_args(&h->cfg, h->capacity, h->chunk_limit, input, target, signal,
                                 send_counts, recv_counts, bias, P, core_num, dtype, nblk,
                                 hidden);
  if (st != A2AV_OK) return st;
  int64_t payload = 0;
  st = a2av::check_host_counts(&h->cfg, host_send_counts, a2av::elem_bytes(dtype),
                               int64_t(nblk) * hidden, 0, &payload);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.nblk = nblk;
  x.bias = bias;
  x.hidden = hidden;
  x.mode = dtype == A2AV_BF16 ? 1 : 2;
  x.launches = a2av::launches_for(payload, h->chunk_limit);
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_run_indexed_host_counts(a2av_handle* h, const void* input, void* target,
                                 int32_t* signal, const int32_t* send_counts,
                                 int32_t* recv_counts, const int32_t* index,
                                 const int32_t* host_send_counts, int32_t P, int64_t core_num,
                                 int32_t dtype, int32_t row_elems, int64_t index_stride,
                                 void* stream) {
  if (!h) return A2AV_ERR_NULLPTR;
  if (!host_send_counts) return A2AV_ERR_NULLPTR;
  int st = a2av::check_indexed_args(&h->cfg, h->capacity, input, target, signal, send_counts,
                                    recv_counts, index, P, core_num, dtype, row_elems,
                                    index_stride);
  if (st != A2AV_OK) return st;
  int64_t payload = 0;
  st = a2av::check_host_counts(&h->cfg, host_send_counts, a2av::elem_bytes(dtype), row_elems,
                               index_stride, &payload);
  if (st != A2AV_OK) return st;
  RunExtras x;
  x.index = index;
  x.index_stride = index_stride;
  x.row_elems = row_elems;
  x.mode = 3;
  x.launches = a2av::launches_for(payload, h->chunk_limit);
  return enqueue_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

int a2av_check_host_counts(const a2av_config* cfg, const int32_t* host_send_counts,
                           int32_t dtype, int64_t* payload_bytes, int32_t* launches) {
  if (!cfg || !host_send_counts || !payload_bytes || !launches) return A2AV_ERR_NULLPTR;
  if (dtype != A2AV_FP32 && dtype != A2AV_INT8) return A2AV_ERR_UNSUPPORTED_DTYPE;
  return a2av_check_host_counts_ex(cfg, host_send_counts, dtype, 1, 0, payload_bytes, launches);
}

int a2av_check_host_counts_ex(const a2av_config* cfg, const int32_t* host_send_counts,
                              int32_t dtype, int64_t unit, int64_t index_stride,
                              int64_t* payload_bytes, int32_t* launches) {
  if (!cfg || !host_send_counts || !payload_bytes || !launches) return A2AV_ERR_NULLPTR;
  if (dtype != A2AV_FP32 && dtype != A2AV_INT8 && dtype != A2AV_FP16 && dtype != A2AV_BF16)
    return A2AV_ERR_UNSUPPORTED_DTYPE;
  if (a2av::check_config(cfg) != A2AV_OK || unit < 1 || index_stride < 0)
    return A2AV_ERR_INVALID_ARGS;
  int64_t payload = 0;
  const int st = a2av::check_host_counts(cfg, host_send_counts, a2av::elem_bytes(dtype), unit,
                                         index_stride, &payload);
  if (st != A2AV_OK) return st;
  const int64_t limit = cfg->chunk_limit_bytes > 0 ? cfg->chunk_limit_bytes
                                                   : a2av::kDefaultChunkLimit;
  *payload_bytes = payload;
  *launches = a2av::launches_for(payload, limit);
  return A2AV_OK;
}

int a2av_query_error(a2av_handle* h) {
  if (!h) return A2AV_ERR_NULLPTR;
  DeviceGuard guard(h->device);
  hipError_t e = hipStreamSynchronize(h->last_stream);
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
  int32_t err = 0;
  e = hipMemcpy(&err, &h->ws.plan->error, sizeof(err), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(h, e, "hipMemcpy(error)");
  if (err != 0) {
    const int32_t zero = 0;
    e = hipMemcpy(&h->ws.plan->error, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(h, e, "hipMemcpy(clear error)");
  }
  return err;
}

int a2av_profile_read(a2av_handle* h, double* k1_us, double* k2_us, int32_t* k2_launches,
                      int32_t* runs) {
  if (!h || !k1_us || !k2_us || !k2_launches || !runs) return A2AV_ERR_NULLPTR;
  if (!h->profile) return A2AV_ERR_INVALID_ARGS;
  DeviceGuard guard(h->device);
  const int64_t n = h->profiled_runs < kProfileRuns ? h->profiled_runs : kProfileRuns;
  double t1 = 0.0, t2 = 0.0;
  int64_t nl = 0;
  for (int64_t k = 0; k < n; ++k) {
    const int64_t run = h->run_counter - 1 - k;
    nl += h->run_launches[size_t(run % kProfileRuns)];
    hipEvent_t* ev = &h->events[size_t(run % kProfileRuns) * size_t(h->events_per_run)];
    hipError_t e = hipEventSynchronize(ev[h->events_per_run - 1]);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventSynchronize");
    float ms1 = 0.f, ms2 = 0.f;
    if ((e = hipEventElapsedTime(&ms1, ev[0], ev[1])) != hipSuccess)
      return hip_fail(h, e, "hipEventElapsedTime");
    if ((e = hipEventElapsedTime(&ms2, ev[1], ev[h->events_per_run - 1])) != hipSuccess)
      return hip_fail(h, e, "hipEventElapsedTime");
    t1 += double(ms1) * 1e3;
    t2 += double(ms2) * 1e3;
  }
  *k1_us = t1;
  *k2_us = t2;
  *k2_launches = int32_t(nl);
  *runs = int32_t(n);
  h->profiled_runs = 0;
  return A2AV_OK;
}

int a2av_profile_sample(a2av_handle* h, int32_t every) {
  if (!h) return A2AV_ERR_NULLPTR;
  if (!h->profile || every < 1) return A2AV_ERR_INVALID_ARGS;
  h->profile_every = every;
  h->enqueued = 0;
  return A2AV_OK;
}

const char* a2av_last_hip_error(a2av_handle* h) { return h ? h->last_error.c_str() : ""; }

}  // extern "C"

// ------------------------------------------------------------------ no-alloc entry point

// The workspace of a2av_run_noalloc: one array per device that the library
// runs on, held until the process ends.  Host code never uses the array's
// name as an address (in host code it is a stand-in, not device memory): the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = 192 * 1024;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct NoallocDevice {
  bool ready = false;
  int status = A2AV_OK;   // set-up outcome (HIP errors are kept)
  char* base = nullptr;   // device address of `scratch` on this device
  int cus = 0;
  int wgs_per_cu = 0;
};

NoallocDevice g_noalloc[kMaxDevices];
std::mutex g_noalloc_mu;

// Set-up on the first call on a device (that device current): the scratch
// array's device address and the copy kernel's co-resident capacity.
const NoallocDevice* noalloc_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoallocDevice& d = g_noalloc[dev];
  if (d.ready) return &d;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
  int per_cu = 0;
  if (e == hipSuccess) e = a2av::copy_occupancy(&per_cu);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    d.status = A2AV_ERR_HIP;
  } else {
    d.base = static_cast<char*>(ptr);
    d.cus = prop.multiProcessorCount;
    d.wgs_per_cu = per_cu;
    d.status = A2AV_OK;
  }
  d.ready = true;
  return &d;
}

}  // namespace

extern "C" {

int a2av_run_noalloc(const void* input, void* target, int32_t* signal,
                     const int32_t* send_counts, int32_t* recv_counts, int32_t* status,
                     int32_t P, int64_t in_slab_bytes, int64_t tgt_slab_bytes, int32_t S,
                     int64_t core_num, int32_t dtype, void* stream) {
  if (!status) return A2AV_ERR_NULLPTR;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return A2AV_ERR_HIP;
  }
  const NoallocDevice* d = noalloc_device(dev);
  if (!d) return A2AV_ERR_INVALID_ARGS;
  if (d->status != A2AV_OK) return d->status;

  a2av_config cfg{};
  cfg.device = dev;
  cfg.P = P;
  cfg.in_slab_bytes = in_slab_bytes;
  cfg.tgt_slab_bytes = tgt_slab_bytes;
  cfg.S = S;
  const int64_t capacity = int64_t(d->wgs_per_cu) * d->cus;
  int st = a2av::check_run_args(&cfg, capacity, input, target, signal, send_counts, recv_counts,
                                P, core_num, dtype);
  if (st != A2AV_OK) return st;
  // The status word is a sixth operand: it may not share a byte with the others.
  const uintptr_t sp = reinterpret_cast<uintptr_t>(status);
  const uintptr_t lo[5] = {uintptr_t(input), uintptr_t(target), uintptr_t(signal),
                           uintptr_t(send_counts), uintptr_t(recv_counts)};
  const uint64_t len[5] = {uint64_t(P) * uint64_t(in_slab_bytes),
                           uint64_t(P) * uint64_t(tgt_slab_bytes), uint64_t(P) * uint64_t(S) * 4u,
                           uint64_t(P) * uint64_t(P) * 4u, uint64_t(P) * uint64_t(P) * 4u};
  for (int i = 0; i < 5; ++i)
    if (sp < lo[i] + len[i] && lo[i] < sp + 4u) return A2AV_ERR_INVALID_ARGS;
  // The workspace must fit the array (P <= 64 and the device's co-resident
  // capacity decide its size).
  if (carve_workspace(nullptr, P, capacity, nullptr, 0) > kScratchBytes)
    return A2AV_ERR_INVALID_ARGS;

  // A handle on the stack: nothing here allocates (its containers stay empty).
  a2av_handle h;
  h.cfg = cfg;
  h.device = dev;
  h.cus = d->cus;
  h.wgs_per_cu = d->wgs_per_cu;
  h.capacity = capacity;
  h.chunk_limit = a2av::kDefaultChunkLimit;
  h.launches = a2av::chunk_launches(&cfg, h.chunk_limit);
  h.spin_limit = kDefaultSpinLimit;
  h.keep_error_text = false;
  h.status_out = status;
  carve_workspace(d->base, P, capacity, &h.ws, 0);
  RunExtras x;
  return enqueue_run(&h, input, target, signal, send_counts, recv_counts, P, core_num, dtype, x,
                     stream);
}

}  // extern "C"
