// kernels.hip -- the two gfx950 kernels of the all_to_all_v exchange.
//
// K1 (count_kernel, one 1024-thread workgroup; the row gather adds up to 63
// more to check its gather lists): checks the count matrix and the signal
// on the device and derives every segment's source and target byte offsets
// (exclusive prefixes along d on the send side and along s on the receive
// side, one wave scanning each row or column of the LDS copy of the matrix
// with DPP lane moves), and the prefix of the flattened payload that K2
// partitions.
//
// K2 (copy_kernel, W = B * G workgroups): the flattened payload is cut into
// tiles of at most 64 KiB (128 KiB for the bias and gather bodies); the first
// eighth is dealt round-robin to the workgroups, the rest are claimed from a
// counter.  Inside a segment the
// copy is destination-aligned: 128-bit streaming buffer loads and
// device-scope streaming buffer stores in the body, numbered from the
// destination's 128-byte line so every wave store writes whole lines, and
// byte stores for the at most 15 bytes at either end, so no byte outside a
// segment is ever written.  When source and destination differ by an odd
// number of bytes mod 4 the body is realigned in registers: each wave loads
// a row of 64 aligned source words, every lane takes its right neighbour's
// word by a DPP lane move and funnels the two with v_alignbyte; a whole
// number of dwords apart, the source is read directly with dword-aligned
// 16-byte loads.  Pieces of at
// most 8 KiB are copied by one wave each, dealt to the waves in turn, so a
// tile of many small segments costs about one memory round trip instead of
// one per segment.  Separate instantiations add the bias (BF16 with an FP32
// bias, FP16 with an FP16 bias) or gather the rows of the indexed exchange.
// The run's final launch writes recv_counts, the transpose of send_counts,
// and every admitted block raises its flag in every
// rank's signal row, and when B > 1 (a cooperative launch) every workgroup
// waits, with a bounded spin, until all B blocks have arrived (polling one
// of several copies of the arrival counter).  The block/flag protocol is the
// block-aware exchange barrier of the PyPTO "LowerL2TensorCollectives Pass"
// page ("Launch width": all admitted blocks co-resident; a refused launch
// rather than a partial one) with per-peer sequence counters as in the start
// barrier of the "vccl alltoallv dev log" page (section 6.1).
#include "a2av.h"
#include "kernels.h"
#include "plan.h"

namespace a2av {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kUnroll = 4;          // 16-byte words in flight per lane, aligned body
constexpr int kRealignUnroll = 4;   // 64-word rows in flight per wave, realigned body

// Flattened payload bytes per workgroup tile: one pass of the body.  64 KiB
// for the byte copy (1024 threads, 4 words per lane) and for the bias body
// (512 threads, 8 words per lane), 128 KiB for the gather body (1024
// threads, 8 words per lane).  With the copy body at 64 KiB tiles c5 ran
// 2,715 -> 2,624 us per run, c3 181.5 -> 176.4, c4 338.5 -> 328.1 (the
// narrower window of tiles in flight streams better, as the probes show);
// at 1024 threads the bias and gather bodies lost 9 % at 64 KiB, and the
// gather body still loses at 512 threads.
template <int MODE>
constexpr int64_t tile_bytes() {
  return MODE == 3 ? 131072 : 65536;
}

// Buffer resources: word 3 of a raw (untyped, stride 0) buffer descriptor on
// the gfx9 family; num_records is in bytes and the hardware drops any access
// past it (loads read 0, stores are discarded), so a piece's descriptor also
// fences its accesses to the piece.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy bits of buffer instructions on gfx950: nt = 2 (streaming),
// sc1 = 16 (device scope).  Payload loads stream; payload stores stream and
// are device-scope, so a store is visible to every XCD once acknowledged and
// the arrival below needs no L2 writeback.
constexpr int kLoadPolicy = 2;
constexpr int kStorePolicy = 2 | 16;

// a / b for b >= 1.  A 64-bit division is a long software sequence on the
// GPU; when both operands are non-negative and fit 32 bits (the usual case
// for row and list positions) the 32-bit one gives the same quotient for a
// fraction of the instructions.  Any other a (a negative count sum among
// them) takes the 64-bit division.
__device__ inline int64_t div_nonneg(int64_t a, int64_t b) {
  if (((uint64_t(a) | uint64_t(b)) >> 32) == 0) return int64_t(uint32_t(a) / uint32_t(b));
  return a / b;
}

// ------------------------------------------------------------------ K1

// The LDS matrices of K1 are indexed [row][column] with a pitch of
// kMaxP + 1 entries, so a wave's lanes walking rows (a stride of one pitch)
// and lanes walking columns (consecutive entries) both hit distinct banks.
constexpr int kPitch = kMaxP + 1;
__device__ inline int lds_at(int r, int c) { return r * kPitch + c; }

// v moved across lanes by one DPP pattern, each 32-bit half on its own;
// lanes the pattern gives no source, or outside kRowMask, read 0.
template <int kCtrl, int kRowMask>
__device__ inline int64_t dpp_move(int64_t v) {
  const uint64_t u = uint64_t(v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(u)), kCtrl, kRowMask, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), kCtrl, kRowMask, 0xf, false);
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Inclusive prefix sum of v over the 64 lanes of a wave (all lanes active):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (row_shr), then the
// last lane of row 0 (and of row 2) is added to row 1 (row 3) and the last
// lane of row 1 to rows 2 and 3 (row_bcast:15, row_bcast:31).
__device__ inline int64_t wave_inclusive_scan(int64_t v) {
  v += dpp_move<0x111, 0xf>(v);
  v += dpp_move<0x112, 0xf>(v);
  v += dpp_move<0x114, 0xf>(v);
  v += dpp_move<0x118, 0xf>(v);
  v += dpp_move<0x142, 0xa>(v);
  v += dpp_move<0x143, 0xc>(v);
  return v;
}

// The same scan on 32-bit values, when every partial sum fits: one DPP add
// per step instead of two moves and a 64-bit add.
__device__ inline int32_t wave_inclusive_scan32(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Inclusive scans of two 32-lane halves of a wave at once (lanes 0-31 and
// 32-63): the row steps, then lane 15 of each half into its upper row; the
// last step, which would carry lane 31 into the upper half, is left out.
__device__ inline int32_t wave_half_scan32(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  return v;
}

// K1's outputs for a valid run, by workgroup 0: the segment tables and the
// cleared counters of the run.
__device__ void write_tables(const CountParams& p, const int32_t* C, int64_t* soff, int64_t* pre,
                             int64_t* doff, const int64_t* rowbase, const int64_t* colbase) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  constexpr int kWaves = kCountThreads / kWave;
  const int P = p.P;
  const int PP = P * P;
  __shared__ int64_t rstride[kMaxP];  // bytes per source block-row

  // The flattened order K2 partitions.  The copy and bias bodies take it
  // destination-major (segment j = d*P + s): the tiles in flight then write
  // one contiguous stretch of a target slab and read pieces of several
  // source slabs, which DRAM serves better than the transpose the other way
  // round.  The row gather takes it source-major (j = s*P + d), measured
  // faster for it.
  const bool dmajor = p.index == nullptr;
  // A column's bytes never exceed tgt_slab, and outside the row gather a
  // row's never exceed in_slab (the capacity checks passed), so below 2^31
  // bytes per slab every partial sum fits a 32-bit scan.  The row gather
  // bounds a row by its gather list instead (rows may repeat), which can
  // pass 2^31 bytes from a small table: it keeps the 64-bit scans.
  const bool narrow = dmajor && p.in_slab < (int64_t(1) << 31) &&
                      p.tgt_slab < (int64_t(1) << 31);
  auto exclusive = [&](int64_t v) -> int64_t {
    return narrow ? int64_t(wave_inclusive_scan32(int32_t(v))) - v : wave_inclusive_scan(v) - v;
  };

  // Send side, one wave per source row s (lane d): the exclusive prefix
  // along d of the row's bytes (input packed by destination) gives the
  // source offsets; with nblk > 1 the source offset is instead the prefix of
  // the sub-block sizes (the segment's sub-block in block-row 0; block-rows
  // are sstride[s] bytes apart).  Receive side, one wave per destination
  // column d (lane s): the exclusive prefix along s (target packed by
  // source).  Each side writes the flattened prefix in its own order.
  // With 32-bit scans and P <= 32 a wave takes two rows (columns) at once,
  // one per 32-lane half.
  const bool pairs = narrow && P <= 32;
  const int half = pairs ? lane >> 5 : 0;
  const int l = pairs ? lane & 31 : lane;
  const int per_wave = pairs ? 2 : 1;
  auto excl = [&](int64_t v) -> int64_t {
    return pairs ? int64_t(wave_half_scan32(int32_t(v))) - v : exclusive(v);
  };
  for (int s0 = wave * per_wave; s0 < P; s0 += kWaves * per_wave) {
    const int s2 = s0 + half;
    const bool on = l < P && s2 < P;
    const int32_t c = on ? C[lds_at(s2, l)] : 0;
    const int64_t v = int64_t(c) * p.elem;
    const int64_t ex = excl(v);
    int64_t sv = v;
    int64_t sex = ex;
    if (p.nblk != 1) {
      sv = int64_t(c / p.nblk) * p.elem;
      sex = excl(sv);
    }
    if (on) {
      soff[lds_at(s2, l)] = int64_t(s2) * p.in_slab + sex;
      if (!dmajor) pre[lds_at(s2, l)] = rowbase[s2] + ex;
    }
    if (l == P - 1 && s2 < P) {
      p.ws.sstride[s2] = sex + sv;
      rstride[s2] = sex + sv;
    }
  }
  for (int d0 = wave * per_wave; d0 < P; d0 += kWaves * per_wave) {
    const int d = d0 + half;
    const bool on = l < P && d < P;
    const int64_t v = on ? int64_t(C[lds_at(l, d)]) * p.elem : 0;
    const int64_t ex = excl(v);
    if (on) {
      doff[lds_at(l, d)] = int64_t(d) * p.tgt_slab + ex;
      if (dmajor) pre[lds_at(d, l)] = colbase[d] + ex;
    }
  }
  __syncthreads();
  if (p.expand) {
    // The blocked byte copy, one segment per sub-block: entry v is sub-block
    // a = v % nblk of destination-major pair j = v / nblk (d = j / P, s = j %
    // P), so K2 copies every piece as in the plain exchange.  The flattened
    // order is the same bytes in the same order as with P * P segments.
    const int nb = p.nblk;
    for (int v = tid; v < PP * nb; v += kCountThreads) {
      const int j = v / nb;
      const int a = v - j * nb;
      const int d = j / P;
      const int s2 = j - d * P;
      const int64_t sub = int64_t(C[lds_at(s2, d)] / nb) * p.elem;
      p.ws.prefix[v] = pre[lds_at(d, s2)] + a * sub;
      p.ws.src_off[v] = soff[lds_at(s2, d)] + a * rstride[s2];
      p.ws.dst_off[v] = doff[lds_at(s2, d)] + a * sub;
    }
  } else {
    for (int i = tid; i < PP; i += kCountThreads) {
      // Flattened segment i is s -> d: i = d*P + s (destination-major) or
      // s*P + d (source-major); pre holds it at lds_at(d, s) or lds_at(s, d).
      const int hi = i / P;
      const int lo = i - hi * P;
      const int s2 = dmajor ? lo : hi;
      const int d = dmajor ? hi : lo;
      p.ws.src_off[i] = soff[lds_at(s2, d)];
      p.ws.prefix[i] = pre[lds_at(hi, lo)];
      p.ws.dst_off[i] = doff[lds_at(s2, d)];
    }
  }
  for (int b = tid; b < p.B; b += kCountThreads) p.ws.blk_cnt[b] = 0u;
  if (tid < kArriveReplicas) p.ws.arrived[int64_t(tid) * kArriveStride] = 0u;
  if (tid == 0) {
    p.ws.prefix[p.expand ? PP * p.nblk : PP] = rowbase[kMaxP];
    p.ws.plan->claim[0] = 0u;
    p.ws.plan->claim[1] = 0u;
  }
}

// The run's verdict.  With one workgroup its flags decide.  Otherwise every
// workgroup adds to one 64-bit word of the plan, in one atomic: 1 to the
// count of workgroups done (bits 0-7) and 1 to the field of each failure
// kind it found (8 bits each: at most 64 workgroups, so no field carries
// into the next).  The add that brings the count to the grid size sees every
// workgroup's findings; that workgroup latches the status or marks the run
// valid, and clears the word for the next run.
__device__ void verdict(const CountParams& p, int f, int64_t total) {
  if (threadIdx.x != 0) return;
  RunPlan* plan = p.ws.plan;
  // Failure kinds (flag bits) and their fields.
  constexpr int kKinds[5] = {1, 2, 4, 8, 16};
  uint64_t mine = 1u;
  for (int k = 0; k < 5; ++k)
    if (f & kKinds[k]) mine += uint64_t(1) << (8 * (k + 1));
  uint64_t all = mine;
  if (gridDim.x > 1) {
    all += __hip_atomic_fetch_add(&plan->kstate, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((all & 0xFFu) != gridDim.x) return;
  }
  int any = 0;
  for (int k = 0; k < 5; ++k)
    if ((all >> (8 * (k + 1))) & 0xFFu) any |= kKinds[k];
  if (any != 0) {
    // Order: negative count, count not whole sub-blocks or rows,
    // over-capacity, gather index outside its table, unequal signal.
    const int code = (any & 1) ? A2AV_ERR_INVALID_ARGS
                   : (any & 8) ? A2AV_ERR_INVALID_ARGS
                   : (any & 2) ? A2AV_ERR_OVER_CAPACITY
                               : A2AV_ERR_INVALID_ARGS;
    atomicCAS(&plan->error, 0, code);
    plan->valid = 0;
    if (p.status_out) *p.status_out = code;
  } else {
    plan->total_bytes = total;
    plan->valid = 1;
    if (p.status_out) *p.status_out = A2AV_OK;
  }
  if (gridDim.x > 1)
    __hip_atomic_store(&plan->kstate, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kCountThreads) void count_kernel(CountParams p) {
  __shared__ int32_t C[kMaxP * kPitch];     // C[lds_at(s, d)] = send_counts[s][d]
  __shared__ int64_t soff[kMaxP * kPitch];  // staged outputs, written back coalesced
  __shared__ int64_t pre[kMaxP * kPitch];
  __shared__ int64_t doff[kMaxP * kPitch];
  __shared__ int64_t rowsum[kMaxP];        // elements (row gather: rows) each source sends
  __shared__ int64_t rowbase[kMaxP + 1];   // bytes before source s (s-major order)
  __shared__ int64_t colbase[kMaxP];       // bytes before destination d (d-major order)
  __shared__ int flags;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  constexpr int kWaves = kCountThreads / kWave;
  const int P = p.P;
  const int PP = P * P;

  if (tid == 0) flags = 0;

  // Row gather: this workgroup's slice of the P x index_stride gather-list
  // entries (flat position e = s * index_stride + k), split evenly among the
  // launch's checking workgroups: all of them when the launch has one,
  // otherwise every workgroup but 0, which writes the tables.  The thread's
  // first kPre entries of it are loaded now, so that their round trip
  // overlaps the counts'; which of them are in use (k below the rows source
  // s sends) is known only once the counts are summed.  Every entry read
  // lies inside the [P, index_stride] lists.
  constexpr int kPre = 8;
  int32_t pre_entry[kPre];
  int64_t g_lo = 0, g_hi = 0;
  if (p.index != nullptr && (gridDim.x == 1 || blockIdx.x != 0)) {
    const int64_t entries = int64_t(P) * p.index_stride;
    const int64_t checkers = gridDim.x == 1 ? 1 : gridDim.x - 1;
    const int64_t slot = gridDim.x == 1 ? 0 : blockIdx.x - 1;
    const int64_t per = (entries + checkers - 1) / checkers;
    g_lo = per * slot < entries ? per * slot : entries;
    g_hi = g_lo + per < entries ? g_lo + per : entries;
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int64_t e = g_lo + tid + int64_t(j) * kCountThreads;
      pre_entry[j] = e < g_hi ? p.index[e] : 0;
    }
  }
  __syncthreads();

  // Load the counts; note negatives (bit 0), counts that are not whole
  // sub-blocks or rows (bit 3: p.unit does not divide them) and a signal that
  // is not uniform over the admitted entries (bit 2).  The loops are unrolled
  // so each thread issues its loads back to back.
  const int64_t unit = p.unit;
  int bad = 0;
#pragma unroll 4
  for (int i = tid; i < PP; i += kCountThreads) {
    const int32_t c = p.send_counts[i];
    C[lds_at(i / P, i - (i / P) * P)] = c;
    bad |= c < 0 ? 1 : 0;
    bad |= (unit > kInt32Max ? c != 0 : c % int32_t(unit) != 0) ? 8 : 0;
  }
  // The signal is checked by workgroup 0 (the others check gather-list
  // slices of the row gather).
  const int32_t base = p.signal[0];
  if (blockIdx.x == 0) {
    for (int r = wave; r < P; r += kWaves) {
      const int32_t* row = p.signal + int64_t(r) * p.S;
#pragma unroll 4
      for (int b = lane; b < p.B; b += kWave) bad |= row[b] != base ? 4 : 0;
    }
  }
  if (bad) atomicOr(&flags, bad);
  __syncthreads();

  // Row sums (what each source sends) in wave 0 and column sums (what each
  // destination receives) in wave 1: lane s (or d) walks its row (column) of
  // the LDS matrix, then the wave scans the byte totals across its lanes into
  // the row bases, the exclusive prefix of the row totals (rowbase[kMaxP] =
  // T), and the column bases, that of the column totals.  Lanes at or past P
  // add nothing.  Then the capacity checks: a source overflows its input
  // slab or, in the indexed exchange, sends more rows than its gather list
  // holds; a destination overflows its target slab.
  if (wave < 2) {
    int64_t acc = 0;
    if (lane < P) {
      if (wave == 0) {
        for (int d = 0; d < P; ++d) acc += C[lds_at(lane, d)];
      } else {
        for (int s2 = 0; s2 < P; ++s2) acc += C[lds_at(s2, lane)];
      }
    }
    const int64_t bytes = acc * p.elem;
    const int64_t incl = wave_inclusive_scan(bytes);
    if (wave == 0) {
      if (lane < P) {
        rowsum[lane] = p.index != nullptr ? div_nonneg(acc, unit) : acc;
        rowbase[lane] = incl - bytes;
        if (p.index != nullptr ? div_nonneg(acc, unit) > p.index_stride : bytes > p.in_slab)
          atomicOr(&flags, 2);
      }
      if (lane == kWave - 1) {
        rowbase[kMaxP] = incl;
        // Never reached when every row and column fits (the launches cover
        // P times the smaller slab, or for the row gather the smaller of P
        // target slabs and P full gather lists).
        if (incl > p.payload_cap) atomicOr(&flags, 2);
      }
    } else if (lane < P) {
      colbase[lane] = incl - bytes;
      if (bytes > p.tgt_slab) atomicOr(&flags, 2);
    }
  }
  __syncthreads();

  // Indexed exchange, counts valid (no negative or partial-row count, no
  // source over its gather list): every gather-list entry in use in this
  // workgroup's slice must name a whole row of its table (bit 4 of the flags
  // word: 16).  The prefetched entries first, then the rest of the slice
  // source by source, loading entries in use only.
  if (p.index != nullptr && (flags & (1 | 2 | 8)) == 0) {
    // Unsigned compare: a negative entry is a huge value.  Entries are int32,
    // so a table of 2^31 rows or more admits every non-negative entry.
    const uint32_t limit = uint32_t(p.table_rows < (int64_t(1) << 31) ? p.table_rows
                                                                      : (int64_t(1) << 31));
    const int64_t stride = p.index_stride;
    const int64_t pre_hi = g_lo + int64_t(kPre) * kCountThreads < g_hi
                               ? g_lo + int64_t(kPre) * kCountThreads
                               : g_hi;
    int bad_row = 0;
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int64_t e = g_lo + tid + int64_t(j) * kCountThreads;
      if (e < pre_hi) {
        const int64_t s2 = div_nonneg(e, stride);
        if (e - s2 * stride < rowsum[s2] && uint32_t(pre_entry[j]) >= limit) bad_row = 16;
      }
    }
    for (int64_t s2 = div_nonneg(pre_hi, stride); pre_hi < g_hi && s2 < P && s2 * stride < g_hi; ++s2) {
      const int64_t k0 = (pre_hi > s2 * stride ? pre_hi : s2 * stride) - s2 * stride;
      const int64_t in_use = rowsum[s2];
      const int64_t k1 = g_hi - s2 * stride < in_use ? g_hi - s2 * stride : in_use;
      const int32_t* list = p.index + s2 * stride;
#pragma unroll 8
      for (int64_t k = k0 + tid; k < k1; k += kCountThreads)
        bad_row |= uint32_t(list[k]) >= limit ? 16 : 0;
    }
    if (bad_row) atomicOr(&flags, bad_row);
    __syncthreads();
  }

  const int f = flags;
  // Workgroup 0 writes the tables and clears the run's counters, then takes
  // part in the verdict; the other workgroups go straight to it.  The tables
  // of a run that fails are never read.
  if (f == 0 && blockIdx.x == 0) write_tables(p, C, soff, pre, doff, rowbase, colbase);
  verdict(p, f, rowbase[kMaxP]);
}
// ------------------------------------------------------------------ K2

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, int64_t word) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, int(word * 16), 0, kLoadPolicy);
}

// The whole offset goes in the vector offset and soffset stays the constant
// 0.  With an SGPR soffset this compiler leaves out the wait states it puts
// between a 128-bit buffer store and a VALU write of the store's data
// registers, and on gfx950 the stores then wrote the new values: a bias body
// that stepped through its words by soffset gave wrong results.
__device__ inline void store16(__amdgpu_buffer_rsrc_t r, int64_t word, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, int(word * 16), 0, kStorePolicy);
}

// Output word = bytes [phi, phi+16) of the 32 bytes a:b, phi = 4*Q + r.
template <int Q>
__device__ inline u32x4 funnel(u32x4 a, u32x4 b, uint32_t r) {
  const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u32x4 o;
  o.x = __builtin_amdgcn_alignbyte(c[Q + 1], c[Q + 0], r);
  o.y = __builtin_amdgcn_alignbyte(c[Q + 2], c[Q + 1], r);
  o.z = __builtin_amdgcn_alignbyte(c[Q + 3], c[Q + 2], r);
  o.w = __builtin_amdgcn_alignbyte(c[Q + 4], c[Q + 3], r);
  return o;
}

// The copy bodies below run on a group of ng threads, ng / kWave waves: the
// whole workgroup (ng = kCopyThreads, t = thread index, gw = wave index) or
// one wave (ng = kWave, t = lane, gw = 0).  The group size is a run-time
// value so that both share one copy of each body (two inlined copies of the
// bodies overflow the 128 registers a 1024-thread workgroup allows).

// Body with the destination 16-byte aligned and the source at least
// dword-aligned: K words.  Thread t
// moves words t, t + ng, ... : each load instruction of a wave covers 1 KiB,
// and a thread's kUnroll loads in flight are ng words apart.
__device__ inline void grp_copy_aligned(const u32x4* s, u32x4* d, int64_t K, int tid, int ng) {
  const int NT = ng;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, K * 16);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(d, K * 16);
  // Words are numbered from the start of the 128-byte destination line that
  // holds word 0 (the lp words before it get k < 0 and are skipped), so each
  // wave's store instruction writes whole lines: a line split between two
  // instructions can reach HBM as two partial writes.
  const int64_t lp = int64_t((reinterpret_cast<uintptr_t>(d) >> 4) & 7u);
  // A predicated pass over words [k0, k0 + NT * kUnroll) of [0, K), so short
  // pieces keep kUnroll loads in flight too.
  auto guarded_pass = [&](int64_t k0) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t k = k0 + j * NT + tid;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (k >= 0 && k < K) v[j] = load16(rs, k);
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t k = k0 + j * NT + tid;
      if (k >= 0 && k < K) store16(rd, k, v[j]);
    }
  };
  int64_t k0 = -lp;
  if (lp != 0) {
    guarded_pass(k0);
    k0 += int64_t(NT) * kUnroll;
  }
  for (; k0 + int64_t(NT) * kUnroll <= K; k0 += int64_t(NT) * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) v[j] = load16(rs, k0 + j * NT + tid);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) store16(rd, k0 + j * NT + tid, v[j]);
  }
  if (k0 < K) guarded_pass(k0);  // the remainder, under NT * kUnroll words
}

// v moved one lane down the wave: lane l receives lane l + 1's value (DPP
// wave_shl:1, which gfx9-family parts such as gfx950 provide); lane 63
// receives 0.
__device__ inline u32x4 wave_shl1(u32x4 v) {
  u32x4 o;
  o.x = uint32_t(__builtin_amdgcn_update_dpp(0, int(v.x), 0x130, 0xf, 0xf, false));
  o.y = uint32_t(__builtin_amdgcn_update_dpp(0, int(v.y), 0x130, 0xf, 0xf, false));
  o.z = uint32_t(__builtin_amdgcn_update_dpp(0, int(v.z), 0x130, 0xf, 0xf, false));
  o.w = uint32_t(__builtin_amdgcn_update_dpp(0, int(v.w), 0x130, 0xf, 0xf, false));
  return o;
}

// Body whose source sits phi = 4*Q + r bytes (r = 1..3) past a 16-byte boundary:
// output word k is bytes [phi, phi+16) of aligned source words A[k], A[k+1].
// Words A[0..K] all hold body bytes, so every load stays inside 16-byte words
// that the segment touches.  Rows of 64 output words go to the group's waves
// in turn, each row one whole 1 KiB run of destination lines: row q holds
// output words k = 64q + l - lp (lp = D's word within its 128-byte line; the
// words with k < 0 are skipped).  Lane l of row q loads A[k], takes A[k + 1]
// from its right neighbour's register by a DPP lane move (no LDS round trip:
// measured 1.5 % faster than exchanging the row through LDS on int8 data at
// odd offsets, 339 -> 334 us per run for 791 MiB at P = 32), and lane 63
// uses A[64q + 64 - lp], which the whole wave loads as one broadcast word.
// One batch of kRealignUnroll rows per wave, starting at row r0.  Guarded
// batches check every word against [0, K]; interior batches (every row whole
// and inside the piece) run unpredicated, so their loads issue back to back.
template <int Q, bool kGuard>
__device__ inline void realign_batch(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rd,
                                     int64_t r0, int64_t nrows, int64_t K, int64_t lp,
                                     uint32_t r, int lane, int wave, int NW) {
  u32x4 v[kRealignUnroll];
  u32x4 x[kRealignUnroll];
#pragma unroll
  for (int j = 0; j < kRealignUnroll; ++j) {
    const int64_t row = r0 + int64_t(j) * NW + wave;
    const int64_t k = row * kWave + lane - lp;
    const int64_t next = row * kWave + kWave - lp;
    if (kGuard) {
      v[j] = u32x4{0u, 0u, 0u, 0u};
      x[j] = u32x4{0u, 0u, 0u, 0u};
      if (row < nrows && k >= 0 && k <= K) v[j] = load16(rs, k);
      if (row < nrows && next <= K) x[j] = load16(rs, next);
    } else {
      v[j] = load16(rs, k);
      x[j] = load16(rs, next);
    }
  }
#pragma unroll
  for (int j = 0; j < kRealignUnroll; ++j) {
    const int64_t row = r0 + int64_t(j) * NW + wave;
    const int64_t k = row * kWave + lane - lp;
    // The right neighbour's word, moved across lanes by DPP (wave_shl:1:
    // lane l reads lane l + 1; every lane of the wave is active here).
    u32x4 hi = wave_shl1(v[j]);
    if (lane == kWave - 1) hi = x[j];
    if (!kGuard || (row < nrows && k >= 0 && k < K)) store16(rd, k, funnel<Q>(v[j], hi, r));
  }
}

template <int Q>
__device__ void grp_copy_realign(const u32x4* A, u32x4* D, int64_t K, uint32_t r,
                                 int lane, int wave, int ng) {
  const int NW = ng / kWave;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(A, (K + 1) * 16);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(D, K * 16);
  const int64_t lp = int64_t((reinterpret_cast<uintptr_t>(D) >> 4) & 7u);
  const int64_t nrows = (K + lp + kWave - 1) / kWave;
  const int64_t batch = int64_t(kRealignUnroll) * NW;
  for (int64_t r0 = 0; r0 < nrows; r0 += batch) {
    // Interior: no row of the batch starts before word 0 (row 0 does when
    // lp > 0) and the last one's next-row word A[64 (r0 + batch) - lp] is
    // inside A[0..K].
    const bool interior = (r0 > 0 || lp == 0) && (r0 + batch) * kWave - lp <= K;
    if (interior)
      realign_batch<Q, false>(rs, rd, r0, nrows, K, lp, r, lane, wave, NW);
    else
      realign_batch<Q, true>(rs, rd, r0, nrows, K, lp, r, lane, wave, NW);
  }
}

// Copy n bytes src -> dst (one piece of one segment) with a group.  The
// destination body is whole aligned 16-byte words; the at most 15 bytes on
// either side are written one byte per thread, so no byte outside the piece
// is ever stored.  Those edge bytes are loaded before the body and stored
// after it, so their round trip overlaps the body's instead of preceding it.
__device__ void grp_copy_piece(const uint8_t* src, uint8_t* dst, int64_t n, int t, int lane,
                               int gw, int ng) {
  const uintptr_t d0 = uintptr_t(dst);
  const uintptr_t body_lo = (d0 + 15u) & ~uintptr_t(15);
  const uintptr_t body_hi = (d0 + uintptr_t(n)) & ~uintptr_t(15);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(dst, n);
  if (body_lo >= body_hi) {
    for (int64_t k = t; k < n; k += ng)
      __builtin_amdgcn_raw_buffer_store_b8(src[k], rb, int(k), 0, kStorePolicy);
    return;
  }
  const int64_t head = int64_t(body_lo - d0);
  const int64_t tail_at = int64_t(body_hi - d0);
  const int64_t tail = n - tail_at;
  // Threads 0..head-1 take the head bytes, threads 16..16+tail-1 the tail.
  const bool edge = t < head || (t >= 16 && t - 16 < tail);
  const int64_t ek = t < 16 ? int64_t(t) : tail_at + t - 16;
  uint8_t ev = 0;
  if (edge) ev = src[ek];

  const uint8_t* sb = src + head;
  const int64_t K = int64_t(body_hi - body_lo) >> 4;
  const uint32_t phi = uint32_t(uintptr_t(sb) & 15u);
  u32x4* D = reinterpret_cast<u32x4*>(dst + head);
  // A source a whole number of dwords past a 16-byte boundary (FP32 data,
  // or any type at such an offset) is read with 16-byte loads at its own,
  // dword-aligned address: the body needs no realignment (measured on c4:
  // 364 -> 352 us per run against a funnel through LDS, and 347.6 -> 340.2
  // against the register funnel below).  Only sources at odd byte phases
  // take the funnel.  A dword-phase wave's 1 KiB load starts mid-line and
  // shares its first and last source lines with the neighbouring waves'
  // loads, which streaming loads sometimes fetch from HBM twice (c4 reads
  // 1.0155x its payload).  Workgroup-scope loads let the neighbours find
  // them in cache (1.0057x) at the same speed back to back, but they keep
  // the source lines in the caches: right after other work has filled the
  // caches with dirty lines, c4 then ran 343 -> 396 us, so the streaming
  // loads stay.
  if ((phi & 3u) == 0) {
    grp_copy_aligned(reinterpret_cast<const u32x4*>(sb), D, K, t, ng);
  } else {
    const u32x4* A = reinterpret_cast<const u32x4*>(sb - phi);
    const uint32_t r = phi & 3u;
    switch (phi >> 2) {
      case 0: grp_copy_realign<0>(A, D, K, r, lane, gw, ng); break;
      case 1: grp_copy_realign<1>(A, D, K, r, lane, gw, ng); break;
      case 2: grp_copy_realign<2>(A, D, K, r, lane, gw, ng); break;
      default: grp_copy_realign<3>(A, D, K, r, lane, gw, ng); break;
    }
  }
  if (edge) __builtin_amdgcn_raw_buffer_store_b8(ev, rb, int(ek), 0, kStorePolicy);
}

// Pieces of at most kSmallPiece bytes (two passes of a wave's aligned body)
// take one wave each, dealt to the waves in turn; `small` counts the small
// pieces met so far and is the same in every wave.  A workgroup copying such
// pieces one after another would pay a memory round trip per piece (measured
// on gfx950: 16 pieces of ~130 bytes took 24 us in one workgroup).  Larger
// pieces take the whole workgroup.
constexpr int64_t kSmallPiece = 8192;

__device__ inline void wg_copy_piece(const uint8_t* src, uint8_t* dst, int64_t n, int tid,
                                     int lane, int wave, int& small) {
  constexpr int NW = kCopyThreads / kWave;
  const bool one = n <= kSmallPiece;
  if (one) {
    const bool mine = (small & (NW - 1)) == __builtin_amdgcn_readfirstlane(wave);
    ++small;
    if (!mine) return;
  }
  // One call site, so the bodies are inlined once.
  grp_copy_piece(src, dst, n, one ? lane : tid, lane, one ? 0 : wave, one ? kWave : kCopyThreads);
}

// ------------------------------------------------ K2, fused bias Add path
//
// BF16 payload with an FP32 bias (MODE 1) or FP16 with an FP16 bias (MODE 2),
// as in the CANN BatchMatMulReduceScatterAllToAll op ("Parameters": the BF16
// case adds in FP32).  Each sum is formed in binary32 and rounded once to
// nearest even by the conversion instruction (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 under the default round-to-nearest-even mode).  For FP16
// the compiler may form the sum with a packed half add instead: binary32
// carries 24 >= 2 * 11 + 2 significand bits, so rounding the binary32 sum to
// binary16 gives the correctly rounded half sum and both forms agree bit for
// bit.

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 16-byte payload words in flight per lane: 8 when each thread keeps one
// column (rows of at most 8192 elements; measured on c5h 1,466 -> 1,381 us of
// K2 per run, with the wait below), 4 when each word loads its own bias
// values (more registers per word).
constexpr int kBiasUnroll = 4;
constexpr int kBiasUnrollShort = 8;

// Reinterpret through a scalar argument: applied directly to an element of an
// ext_vector_type value (b.y), this compiler's __builtin_bit_cast reads
// element 0 whatever the index (seen in the gfx950 code it emits).
__device__ inline float f32_bits(uint32_t u) { return __builtin_bit_cast(float, u); }

// A value every lane of the wave holds, moved to scalar registers (the
// compiler cannot see that values read from LDS at a uniform index are
// uniform, and would otherwise loop over lanes for every buffer access).
__device__ inline int64_t wave_uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

template <typename T>
__device__ inline T* wave_uniform(T* p) {
  return reinterpret_cast<T*>(wave_uniform(int64_t(reinterpret_cast<uintptr_t>(p))));
}

__device__ inline uint32_t add_bf16x2(uint32_t x, float b0, float b1) {
  // bf16 -> f32 is exact: the bits move to the high half.
  f32x2 v;
  v.x = __builtin_bit_cast(float, x << 16) + b0;
  v.y = __builtin_bit_cast(float, x & 0xFFFF0000u) + b1;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline uint32_t add_f16x2(uint32_t x, uint32_t b) {
  const f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, x), f32x2) +
                  __builtin_convertvector(__builtin_bit_cast(f16x2, b), f32x2);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// One 16-byte payload word (8 elements of one row) plus the 8 bias values of
// its columns: two 16-byte bias words for FP32, one for FP16.
template <int MODE>
__device__ inline u32x4 add_bias_word(u32x4 x, u32x4 b0, u32x4 b1) {
  u32x4 o;
  if constexpr (MODE == 1) {
    o.x = add_bf16x2(x.x, f32_bits(b0.x), f32_bits(b0.y));
    o.y = add_bf16x2(x.y, f32_bits(b0.z), f32_bits(b0.w));
    o.z = add_bf16x2(x.z, f32_bits(b1.x), f32_bits(b1.y));
    o.w = add_bf16x2(x.w, f32_bits(b1.z), f32_bits(b1.w));
  } else {
    o.x = add_f16x2(x.x, b0.x);
    o.y = add_f16x2(x.y, b0.y);
    o.z = add_f16x2(x.z, b0.z);
    o.w = add_f16x2(x.w, b0.w);
  }
  return o;
}

// A piece of n bytes (whole 16-byte words, source and destination 16-byte
// aligned: the host checks and the device count check guarantee it) inside
// one sub-block.  Its first element is element e0 of the sub-block, whose
// rows are `hidden` elements long (hidden a multiple of 8, so a word never
// straddles two rows); brow is the sub-block's bias row.
//
// Rows of Hw = hidden / 8 words.  When Hw <= NT the workgroup steps through
// the piece NTe = (NT / Hw) * Hw words at a time (the last NT - NTe threads
// idle), so every thread meets the same column on every step and loads its 8
// bias values once per piece.  Longer rows step NT words at a time and each
// word loads its own bias values; the column then advances by 8 * NT
// (mod hidden) per step.
template <int NT, int MODE>
__device__ void wg_bias_piece(const uint8_t* src, uint8_t* dst, int64_t n, const uint8_t* brow,
                              int64_t e0, int32_t hidden, int tid) {
  constexpr int BE = MODE == 1 ? 4 : 2;  // bias bytes per element
  src = wave_uniform(src);
  dst = wave_uniform(dst);
  brow = wave_uniform(brow);
  n = wave_uniform(n);
  e0 = wave_uniform(e0);
  const int64_t K = n >> 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, n);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst, n);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(brow, int64_t(hidden) * BE);
  const uint32_t H = uint32_t(hidden);
  const uint32_t Hw = H / 8u;
  const int64_t e_t = e0 + 8 * int64_t(tid);
  uint32_t h = uint32_t(e_t - div_nonneg(e_t, int64_t(H)) * int64_t(H));

  if (Hw <= uint32_t(NT)) {
    const int NTe = int((uint32_t(NT) / Hw) * Hw);
    if (tid >= NTe) return;
    const u32x4 b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, int(h * BE), 0, 0);
    u32x4 b1 = u32x4{0u, 0u, 0u, 0u};
    if constexpr (MODE == 1) b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, int(h * BE + 16), 0, 0);
    // Whole steps unpredicated, so a step's loads issue back to back; then
    // the remainder predicated.  The first step is written out ahead of the
    // loop: its payload loads follow the bias loads at once, and its first
    // wait (for the first payload word) covers the bias too.  Inside a loop
    // the compiler's wait for the bias values sat in the loop header, where
    // it made each step wait for the previous step's stores before issuing
    // its loads.
    // A piece lies inside one tile (at most 128 KiB and 127 bytes), so its
    // word counts fit 32 bits; kept there, the step tests stay on the scalar
    // unit instead of borrowing vector registers that the previous step's
    // stores still read (which made each step wait for those stores).
    const int32_t K32 = int32_t(K);
    const int32_t step = NTe * kBiasUnrollShort;
    int32_t k0 = 0;
    if (step <= K32) {
      u32x4 v[kBiasUnrollShort];
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j) v[j] = load16(rs, j * NTe + tid);
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j)
        store16(rd, j * NTe + tid, add_bias_word<MODE>(v[j], b0, b1));
      k0 = step;
    }
    for (; k0 + step <= K32; k0 += step) {
      u32x4 v[kBiasUnrollShort];
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j) v[j] = load16(rs, k0 + j * NTe + tid);
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j)
        store16(rd, k0 + j * NTe + tid, add_bias_word<MODE>(v[j], b0, b1));
    }
    if (k0 < K32) {
      u32x4 v[kBiasUnrollShort];
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j) {
        const int32_t k = k0 + j * NTe + tid;
        v[j] = u32x4{0u, 0u, 0u, 0u};
        if (k < K32) v[j] = load16(rs, k);
      }
#pragma unroll
      for (int j = 0; j < kBiasUnrollShort; ++j) {
        const int32_t k = k0 + j * NTe + tid;
        if (k < K32) store16(rd, k, add_bias_word<MODE>(v[j], b0, b1));
      }
    }
    return;
  }

  const uint32_t inc = uint32_t((8u * NT) % H);
  for (int64_t k0 = 0; k0 < K; k0 += int64_t(NT) * kBiasUnroll) {
    u32x4 v[kBiasUnroll];
    u32x4 b0[kBiasUnroll];
    u32x4 b1[kBiasUnroll];
#pragma unroll
    for (int j = 0; j < kBiasUnroll; ++j) {
      const int64_t k = k0 + j * NT + tid;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      b0[j] = u32x4{0u, 0u, 0u, 0u};
      b1[j] = u32x4{0u, 0u, 0u, 0u};
      if (k < K) {
        v[j] = load16(rs, k);
        b0[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, int(h * BE), 0, 0);
        if constexpr (MODE == 1) b1[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, int(h * BE + 16), 0, 0);
      }
      h += inc;
      if (h >= H) h -= H;
    }
#pragma unroll
    for (int j = 0; j < kBiasUnroll; ++j) {
      const int64_t k = k0 + j * NT + tid;
      if (k < K) store16(rd, k, add_bias_word<MODE>(v[j], b0[j], b1[j]));
    }
  }
}

// ------------------------------------------------ K2, indexed (row gather) path
//
// The indexed exchange reads row j of segment s -> d from table row
// list[j] of source s.  With rows and operands 16-byte aligned every piece
// is whole words on both sides; thread t handles words t, t + NT, ... of the
// piece, keeping its (row, byte-in-row) position and advancing it by NT
// words per word.  A pass of kGatherUnroll words per thread issues its
// gather-list loads back to back (the lanes of a wave share one or two
// entries, so they are broadcasts from cache), then the payload loads, then
// the stores.  Whole passes run unpredicated; only the last pass of a piece
// checks each word, and there the row of a word past the piece is clamped
// to the piece's last row, so every list load stays among the entries in
// use.  (With each list load and its use inside a per-word branch, the
// compiler waited for every list load in turn: eight round trips a pass.)
constexpr int kGatherUnroll = 8;

__device__ void wg_gather_words(const uint8_t* table, uint8_t* dseg, int64_t off0, int64_t n,
                                const int32_t* list, int64_t RB, int tid) {
  constexpr int NT = kCopyThreads;
  table = wave_uniform(table);
  dseg = wave_uniform(dseg);
  list = wave_uniform(list);
  off0 = wave_uniform(off0);
  n = wave_uniform(n);
  RB = wave_uniform(RB);
  const int64_t K = n >> 4;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dseg + off0, n);
  const int64_t step_r = div_nonneg(int64_t(NT) * 16, RB);
  const int64_t step_w = int64_t(NT) * 16 - step_r * RB;
  const int64_t last_row = div_nonneg(off0 + n - 1, RB);
  const int64_t off = off0 + 16 * int64_t(tid);
  int64_t r = div_nonneg(off, RB);
  int64_t w = off - r * RB;
  auto pass = [&](int64_t k0, bool guard) {
    int64_t rw[kGatherUnroll];
    int32_t row[kGatherUnroll];
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      rw[j] = w;
      row[j] = list[guard && r > last_row ? last_row : r];
      w += step_w;
      r += step_r;
      if (w >= RB) {
        w -= RB;
        ++r;
      }
    }
    u32x4 v[kGatherUnroll];
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const int64_t k = k0 + int64_t(j) * NT + tid;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      const u32x4* p = reinterpret_cast<const u32x4*>(table + int64_t(row[j]) * RB + rw[j]);
      if (!guard || k < K) v[j] = __builtin_nontemporal_load(p);
    }
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const int64_t k = k0 + int64_t(j) * NT + tid;
      if (!guard || k < K) store16(rd, k, v[j]);
    }
  };
  int64_t k0 = 0;
  for (; k0 + int64_t(NT) * kGatherUnroll <= K; k0 += int64_t(NT) * kGatherUnroll) pass(k0, false);
  if (k0 < K) pass(k0, true);
}

// wg_gather_words with 32-bit positions, the table read through a buffer
// descriptor with 32-bit offsets: for tables below 2 GiB and pieces that end
// below 2 GiB into their segment (c3i's token tables are 28 MiB).  The
// row/byte bookkeeping per word is then 32-bit arithmetic, and the payload
// address one multiply-add.  Every table offset is row * RB + w with row a
// checked gather entry (below the table's rows) and w < RB, so it stays
// inside the descriptor's range.
__device__ void wg_gather_words32(const uint8_t* table, int64_t table_bytes, uint8_t* dseg,
                                  int64_t off0_, int64_t n_, const int32_t* list, int64_t RB_,
                                  int tid) {
  constexpr uint32_t NT = kCopyThreads;
  table = wave_uniform(table);
  dseg = wave_uniform(dseg);
  list = wave_uniform(list);
  const uint32_t off0 = uint32_t(wave_uniform(off0_));
  const uint32_t n = uint32_t(wave_uniform(n_));
  const uint32_t RB = uint32_t(wave_uniform(RB_));
  const uint32_t K = n >> 4;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dseg + off0, n);
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, wave_uniform(table_bytes));
  const uint32_t step_r = (NT * 16u) / RB;
  const uint32_t step_w = NT * 16u - step_r * RB;
  const uint32_t last_row = (off0 + n - 1u) / RB;
  const uint32_t off = off0 + 16u * uint32_t(tid);
  uint32_t r = off / RB;
  uint32_t w = off - r * RB;
  auto pass = [&](uint32_t k0, bool guard) {
    uint32_t rw[kGatherUnroll];
    uint32_t row[kGatherUnroll];
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      rw[j] = w;
      row[j] = uint32_t(list[guard && r > last_row ? last_row : r]);
      w += step_w;
      r += step_r;
      if (w >= RB) {
        w -= RB;
        ++r;
      }
    }
    u32x4 v[kGatherUnroll];
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const uint32_t k = k0 + uint32_t(j) * NT + uint32_t(tid);
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (!guard || k < K)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rt, int(row[j] * RB + rw[j]), 0, kLoadPolicy);
    }
#pragma unroll
    for (int j = 0; j < kGatherUnroll; ++j) {
      const uint32_t k = k0 + uint32_t(j) * NT + uint32_t(tid);
      if (!guard || k < K) store16(rd, k, v[j]);
    }
  };
  uint32_t k0 = 0;
  for (; k0 + NT * kGatherUnroll <= K; k0 += NT * kGatherUnroll) pass(k0, false);
  if (k0 < K) pass(k0, true);
}

// Source rank of flattened segment i (the order K1 chose for the body).
template <int MODE>
__device__ inline int source_of(int i, int P) {
  return MODE == 3 ? i / P : i % P;
}

// Segment tables of one run, staged in LDS by every workgroup.
struct SegTables {
  int64_t prefix[kMaxP * kMaxP + 1];
  int64_t src[kMaxP * kMaxP];
  int64_t dst[kMaxP * kMaxP];
  int64_t sstride[kMaxP];  // bytes per source block-row (blocked exchange)
  // prefix[64 k] for 64 k <= nseg, side by side: the first level of the
  // whole-wave search reads it with consecutive lanes (prefix itself, read
  // 64 entries apart, put every lane on the same LDS bank).
  int64_t coarse[kWave];
};

// Largest segment i in [0, nseg) with prefix[i] <= x (prefix[0] = 0 <= x),
// by one lane on its own (binary search over the LDS prefix).
__device__ inline int seg_of(const int64_t* prefix, int nseg, int64_t x) {
  int lo = 0;
  int hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same for a wave-uniform x, found by the wave's 64 lanes together: each
// level reads one entry per lane (64 candidates), and the ballot of "entry
// <= x", true on a leading run of lanes since the prefix never falls, gives
// the next base.  One LDS round trip per level of 64 (nseg <= 4096: at most
// two) where the binary search takes up to 12 in turn; the first level reads
// the side-by-side copy of every 64th entry.  All lanes of the wave must be
// active.
__device__ inline int wave_seg_of(const SegTables& t, int nseg, int64_t x, int lane) {
  int base = 0;
  if (nseg > kWave) {
    const bool le = lane * kWave < nseg && t.coarse[lane] <= x;
    base = (__builtin_popcountll(__builtin_amdgcn_ballot_w64(le)) - 1) * kWave;
  }
  const int i = base + lane;
  const bool le = i < nseg && t.prefix[i] <= x;
  return base + __builtin_popcountll(__builtin_amdgcn_ballot_w64(le)) - 1;
}

// A tile boundary x moved forward (never past its segment's end or c_hi) so
// that the destination byte it maps to starts a 128-byte line: neighbouring
// tiles then never share a destination line inside a segment.  Monotone in x.
__device__ inline int64_t align_boundary(const SegTables& t, int nseg, const uint8_t* target,
                                         int64_t x, int64_t c_hi) {
  const int i = seg_of(t.prefix, nseg, x);
  const uintptr_t a = uintptr_t(target) + uintptr_t(t.dst[i] + (x - t.prefix[i]));
  int64_t y = x + int64_t((0u - a) & 127u);
  if (y > t.prefix[i + 1]) y = t.prefix[i + 1];
  if (y > c_hi) y = c_hi;
  return y;
}

// align_boundary for a wave-uniform x (the claimed tiles' bounds), searched
// by the whole wave.
__device__ inline int64_t align_boundary_w(const SegTables& t, int nseg, const uint8_t* target,
                                           int64_t x, int64_t c_hi, int lane, int& seg) {
  const int i = wave_seg_of(t, nseg, x, lane);
  const uintptr_t a = uintptr_t(target) + uintptr_t(t.dst[i] + (x - t.prefix[i]));
  int64_t y = x + int64_t((0u - a) & 127u);
  if (y > t.prefix[i + 1]) y = t.prefix[i + 1];
  if (y > c_hi) y = c_hi;
  seg = i;
  return y;
}

__device__ inline int64_t readlane64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(uint64_t(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(v) >> 32), lane);
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Bounds [a, b) and first segment of static tile t of a launch over the
// flattened bytes [c_lo, c_hi) cut into tiles of `tile` bytes; t < nstatic.
__device__ inline void tile_bounds(const SegTables& tab, int nseg, const uint8_t* target,
                                   int64_t c_lo, int64_t c_hi, int64_t tile, int64_t t,
                                   int64_t& a, int64_t& b, int& i) {
  const int64_t x0 = c_lo + t * tile;
  const int64_t x1 = x0 + tile < c_hi ? x0 + tile : c_hi;
  a = t == 0 ? c_lo : align_boundary(tab, nseg, target, x0, c_hi);
  b = x1 >= c_hi ? c_hi : align_boundary(tab, nseg, target, x1, c_hi);
  i = a < b ? seg_of(tab.prefix, nseg, a) : 0;
}

// Copy the flattened bytes [x, b) that start in segment i, piece by piece.
// The target side of a segment is contiguous.  In the blocked exchange the
// source side is nblk sub-blocks, sub-block a at tab.src[i] + a * sstride[s],
// so a piece is also cut where a sub-block ends (the byte copy gets each
// sub-block as a segment of its own when the tables hold them, and then
// arrives here with nblk = 1).
template <int NT, int MODE>
__device__ inline void copy_range(const CopyParams& p, const SegTables& tab, int64_t x, int64_t b,
                                  int i, int tid, int lane, int wave, int& small) {
  while (x < b) {
    const int64_t seg_lo = tab.prefix[i];
    const int64_t seg_hi = tab.prefix[i + 1];
    if (seg_hi > x) {
      const int64_t pe = b < seg_hi ? b : seg_hi;
      if constexpr (MODE == 3) {
        // Row gather: the segment's rows start at row (src - s * in_slab) / RB
        // of source s's gather list.
        const int s = source_of<MODE>(i, p.P);
        const int64_t RB = p.row_bytes;
        const int64_t row0 = div_nonneg(tab.src[i] - int64_t(s) * p.in_slab, RB);
        const int32_t* list = p.index + int64_t(s) * p.index_stride + row0;
        const uint8_t* table = p.input + int64_t(s) * p.in_slab;
        uint8_t* dseg = p.target + tab.dst[i];
        if (p.gather_words) {
          if (p.in_slab < (int64_t(1) << 31) && pe - seg_lo < (int64_t(1) << 31))
            wg_gather_words32(table, p.in_slab, dseg, x - seg_lo, pe - x, list, RB, tid);
          else
            wg_gather_words(table, dseg, x - seg_lo, pe - x, list, RB, tid);
        } else {
          // Any alignment: one piece per row (or part of a row), copied by
          // the byte-exact path.
          for (int64_t off = x - seg_lo; off < pe - seg_lo;) {
            const int64_t r = div_nonneg(off, RB);
            const int64_t w = off - r * RB;
            const int64_t end = (r + 1) * RB < pe - seg_lo ? (r + 1) * RB : pe - seg_lo;
            const int64_t row = __builtin_amdgcn_readfirstlane(list[r]);
            wg_copy_piece(wave_uniform(table + row * RB + w), wave_uniform(dseg + off),
                          wave_uniform(end - off), tid, lane, wave, small);
            off = end;
          }
        }
      } else if constexpr (MODE != 0) {
        // Fused bias Add: pieces end at sub-block ends; sub-block a of source
        // s takes bias row (s, a).
        const int64_t sub = (seg_hi - seg_lo) / p.nblk;
        const int s = source_of<MODE>(i, p.P);
        const int64_t stride = tab.sstride[s];
        constexpr int be = MODE == 1 ? 4 : 2;
        for (int64_t off = x - seg_lo; off < pe - seg_lo;) {
          const int64_t a = div_nonneg(off, sub);
          const int64_t w = off - a * sub;
          const int64_t end = (a + 1) * sub < pe - seg_lo ? (a + 1) * sub : pe - seg_lo;
          const uint8_t* brow = static_cast<const uint8_t*>(p.bias) +
                                (int64_t(s) * p.nblk + a) * p.hidden * be;
          const uint8_t* src = p.input + tab.src[i] + a * stride + w;
          uint8_t* dst = p.target + tab.dst[i] + off;
          wg_bias_piece<NT, MODE>(src, dst, end - off, brow, w >> 1, p.hidden, tid);
          off = end;
        }
      } else if (p.nblk == 1) {
        const int64_t off = x - seg_lo;
        wg_copy_piece(p.input + tab.src[i] + off, p.target + tab.dst[i] + off, pe - x, tid,
                      lane, wave, small);
      } else {
        const int64_t sub = (seg_hi - seg_lo) / p.nblk;
        const int64_t stride = tab.sstride[source_of<MODE>(i, p.P)];
        for (int64_t off = x - seg_lo; off < pe - seg_lo;) {
          const int64_t a = div_nonneg(off, sub);
          const int64_t w = off - a * sub;
          const int64_t end = (a + 1) * sub < pe - seg_lo ? (a + 1) * sub : pe - seg_lo;
          wg_copy_piece(p.input + tab.src[i] + a * stride + w, p.target + tab.dst[i] + off,
                        end - off, tid, lane, wave, small);
          off = end;
        }
      }
      x = pe;
    }
    ++i;
  }
}

// One K2 launch copies the flattened payload bytes [c_lo, c_hi) of the run.
// The range is cut into tiles of at most tile_bytes<MODE>(), handed out in tile order
// (round-robin first, then by claim), so at any moment the grid streams
// through one narrow window of the source and of the destination (measured
// on gfx950: contiguous per-workgroup ranges that fan out to destination
// slabs 1 GiB apart ran at ~4.1 TB/s, the same bytes as interleaved tiles at
// ~5.6 TB/s).  Every wave derives the same tile bounds and pieces from the
// LDS tables, so static tiles need no workgroup barrier.
template <int NT, int MODE>
__global__ __launch_bounds__(NT) void copy_kernel(CopyParams p) {
  __shared__ SegTables tab;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  RunPlan* plan = p.ws.plan;
  const int nseg = p.nseg;
  auto stage_tables = [&]() {
    for (int i = tid; i <= nseg; i += NT) tab.prefix[i] = p.ws.prefix[i];
    for (int i = tid; i < nseg; i += NT) {
      tab.src[i] = p.ws.src_off[i];
      tab.dst[i] = p.ws.dst_off[i];
    }
    if (tid < p.P) tab.sstride[tid] = p.ws.sstride[tid];
    if (tid < kWave && tid * kWave < nseg) tab.coarse[tid] = p.ws.prefix[tid * kWave];
  };
  // The flag and the payload size are loaded together (one round trip).  The
  // final launch has payload whenever the run has any, so it stages the
  // segment tables in the same round trip; earlier launches first learn
  // whether their chunk holds payload.
  const int valid = plan->valid;
  const int64_t T = plan->total_bytes;
  if (p.last) stage_tables();
  if (valid == 0) return;  // the run failed its device checks: write nothing

  // Launch c claims tiles on plan->claim[c & 1]; the launch before it in the
  // stream (c + 1) has finished with the other counter, which launch c - 1
  // will use: clear it now.  K1 cleared both for the run's first launch.
  if (tid == 0 && blockIdx.x == 0)
    __hip_atomic_store(&plan->claim[(p.chunk + 1) & 1], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);

  const int64_t c_lo = p.chunk_lo < T ? p.chunk_lo : T;
  const int64_t c_hi = p.chunk_hi < T ? p.chunk_hi : T;
  // A chunk past the run's payload has nothing to copy (the final launch
  // still arrives, even with no payload).
  if (c_lo >= c_hi && !p.last) return;
  if (!p.last) stage_tables();
  __syncthreads();
  // The final launch writes recv_counts[d][s] = send_counts[s][d] (entry
  // d*P + s): the run's checks have passed, so a run that fails them, or whose
  // launches fail before the final one is enqueued, leaves it untouched.
  if (p.last && blockIdx.x == 0)
    for (int i = tid; i < p.P * p.P; i += NT)
      p.recv_counts[i] = p.send_counts[(i % p.P) * p.P + i / p.P];

  // Tile size: at most tile_bytes<MODE>(), chosen so W workgroups take the
  // same number of rounds (with the static deal, no workgroup is left with
  // one extra tile).
  constexpr int64_t kTile = tile_bytes<MODE>();
  const int64_t len = c_hi - c_lo;
  const int64_t W = gridDim.x;
  const int64_t rounds = (len + W * kTile - 1) / (W * kTile);
  const int64_t tile = rounds > 0 ? ((len + W * rounds - 1) / (W * rounds) + 15) & ~int64_t(15) : 1;
  const int64_t ntiles = (len + tile - 1) / tile;
  // The first eighth of the rounds (rounded up) is dealt statically: tile t
  // to workgroup t mod W.  The rest go to whichever workgroup asks first, so
  // workgroups that stream slower take fewer tiles and the launch ends when
  // the last tile does, not when the slowest workgroup's share does
  // (measured on gfx950: c5 5.79 -> 6.11 TB/s in-kernel, c3 5.25 -> 5.75;
  // an eighth static rather than a quarter, c5 -0.7 %, c5b -0.6 %; the row
  // gather with its current body, 193.6 -> 191.0 us per run against claiming
  // every tile).
  const int64_t rounds_static = (rounds + 7) / 8;
  const int64_t nstatic = W * rounds_static < ntiles ? W * rounds_static : ntiles;

  int small = 0;  // small pieces met so far (see wg_copy_piece)

  // A wave works through its workgroup's static tiles (blockIdx.x, + W, ...)
  // 64 at a time: lane l first finds the bounds and first segment of the l-th
  // tile of the batch, then the wave walks the batch, reading them with
  // readlane.
  for (int64_t t0 = blockIdx.x; t0 < nstatic; t0 += int64_t(kWave) * W) {
    const int64_t tl = t0 + int64_t(lane) * W;
    int64_t la = 0;
    int64_t lb = 0;
    int li = 0;
    if (tl < nstatic) tile_bounds(tab, nseg, p.target, c_lo, c_hi, tile, tl, la, lb, li);
    for (int j = 0; j < kWave && t0 + int64_t(j) * W < nstatic; ++j) {
      copy_range<NT, MODE>(p, tab, readlane64(la, j), readlane64(lb, j), __builtin_amdgcn_readlane(li, j),
                 tid, lane, wave, small);
    }
  }

  // Claimed tiles: thread 0 asks for the next tile while the workgroup copies
  // the current one.  Claims only grow, so every workgroup leaves the loop
  // once they pass ntiles, and each tile is copied exactly once.
  if (nstatic < ntiles) {
    // The claimed tiles' bounds are wave-uniform, so each wave finds their
    // segments with the whole-wave search, and the claims alternate between
    // two LDS slots, so one barrier per tile suffices (with the binary
    // search and two barriers per tile the 64 KiB tiles ran slower than
    // 128 KiB ones).
    __shared__ int64_t s_claim[2];
    uint32_t* ctr = &plan->claim[p.chunk & 1];
    if (tid == 0)
      s_claim[0] = nstatic + int64_t(__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    int64_t t = s_claim[0];
    int slot = 0;
    while (t < ntiles) {
      uint32_t next = 0;
      if (tid == 0) next = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int64_t x0 = c_lo + t * tile;
      const int64_t x1 = x0 + tile < c_hi ? x0 + tile : c_hi;
      // The segment that holds a: the one x0 lies in, unless a was moved to
      // that segment's end (or the tile is the launch's first).
      int ia = 0;
      int ib = 0;
      const int64_t a = t == 0 ? c_lo : align_boundary_w(tab, nseg, p.target, x0, c_hi, lane, ia);
      const int64_t b = x1 >= c_hi ? c_hi : align_boundary_w(tab, nseg, p.target, x1, c_hi, lane, ib);
      if (t == 0 || a >= tab.prefix[ia + 1]) ia = wave_seg_of(tab, nseg, a, lane);
      if (a < b)
        copy_range<NT, MODE>(p, tab, wave_uniform(a), wave_uniform(b),
                         __builtin_amdgcn_readfirstlane(ia), tid, lane, wave, small);
      // The next claim goes to the other slot: every thread read it at the
      // start of the previous tile, before the barrier that ended that tile.
      if (tid == 0) s_claim[slot ^ 1] = nstatic + int64_t(next);
      __syncthreads();
      slot ^= 1;
      t = s_claim[slot];
    }
  }

  if (!p.last) return;

  // Arrival.  Every payload store is device-scope, so once a wave's stores are
  // acknowledged (vmcnt 0) they are visible to every XCD: that wait is the
  // release.  Then the last workgroup of block b raises signal[r][b] for
  // every rank r and counts the block as arrived; the asm's memory clobber
  // and the barrier keep the compiler from hoisting the atomics above it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave == 0) {
    const int b = int(blockIdx.x) / p.G;
    // A block of one workgroup needs no count (and saves its round trip).
    uint32_t done = 0u;
    if (lane == 0 && p.G != 1)
      done = __hip_atomic_fetch_add(&p.ws.blk_cnt[b], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done == uint32_t(p.G - 1)) {
      // One lane per rank raises the flags, one lane per copy counts the
      // block, each a single wave-wide atomic.
      for (int r = lane; r < p.P; r += kWave)
        __hip_atomic_fetch_add(&p.signal[int64_t(r) * p.S + b], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      for (int k = lane; k < kArriveReplicas; k += kWave)
        __hip_atomic_fetch_add(&p.ws.arrived[int64_t(k) * kArriveStride], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (p.wait && lane == 0) {
      // All admitted blocks are co-resident (cooperative launch); wait until
      // every one has arrived.  Polls are relaxed device-scope loads (no
      // cache invalidation per poll); nothing is read after the wait.  The
      // wait is bounded: a lost arrival latches TIMEOUT instead of hanging.
      const uint32_t* mine =
          p.ws.arrived + int64_t(blockIdx.x % kArriveReplicas) * kArriveStride;
      int spins = 0;
      while (__hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < uint32_t(p.B)) {
        if (++spins > p.spin_limit) {
          int expected = 0;
          __hip_atomic_compare_exchange_strong(&plan->error, &expected, int(A2AV_ERR_TIMEOUT),
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          if (p.status_out)
            __hip_atomic_store(p.status_out, int(A2AV_ERR_TIMEOUT), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  __syncthreads();
}

}  // namespace

hipError_t launch_count(const CountParams& p, int workgroups, hipStream_t stream) {
  // The launch's own status (hipGetLastError could report an earlier call's).
  void* args[] = {const_cast<CountParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&count_kernel), dim3(workgroups),
                         dim3(kCountThreads), args, 0, stream);
}

namespace {

// One instantiation per body, so the plain kernel carries no bias code.
const void* copy_kernel_for(int mode) {
  switch (mode) {
    case 1: return reinterpret_cast<const void*>(&copy_kernel<kBiasThreads, 1>);
    case 2: return reinterpret_cast<const void*>(&copy_kernel<kBiasThreads, 2>);
    case 3: return reinterpret_cast<const void*>(&copy_kernel<kCopyThreads, 3>);
    default: return reinterpret_cast<const void*>(&copy_kernel<kCopyThreads, 0>);
  }
}

int copy_threads_for(int mode) { return mode == 1 || mode == 2 ? kBiasThreads : kCopyThreads; }

}  // namespace

hipError_t launch_copy(const CopyParams& p, int workgroups, bool cooperative, hipStream_t stream) {
  void* args[] = {const_cast<CopyParams*>(&p)};
  const void* f = copy_kernel_for(p.mode);
  if (cooperative)
    return hipLaunchCooperativeKernel(f, dim3(workgroups), dim3(copy_threads_for(p.mode)), args,
                                      0, stream);
  return hipLaunchKernel(f, dim3(workgroups), dim3(copy_threads_for(p.mode)), args, 0, stream);
}

hipError_t copy_occupancy(int* wgs_per_cu) {
  // The largest of the instantiations decides (they share the LDS
  // footprint; register counts differ).
  int best = 1 << 30;
  for (int mode = 0; mode < 4; ++mode) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, copy_kernel_for(mode),
                                                                      copy_threads_for(mode), 0);
    if (e != hipSuccess) return e;
    if (n < best) best = n;
  }
  *wgs_per_cu = best;
  return hipSuccess;
}

}  // namespace a2av
