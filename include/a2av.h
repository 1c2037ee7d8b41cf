/*
 * a2av.h -- C ABI of the MI355X (gfx950) variable-count all-to-all exchange.
 *
 * The operation is the five-operand all_to_all_v of the PyPTO
 * "LowerL2TensorCollectives Pass" page (section "Behavior": operands input,
 * target, signal, send_counts, recv_counts with directions In, InOut, InOut,
 * In, InOut, plus the launch request core_num).  On one GPU the P ranks are
 * virtual: each owns one slab of a shared allocation, and the exchange is an
 * on-device scatter/transpose of segments:
 *
 *   for every source s and destination d (element size e: fp32 4, int8 1)
 *     target[d*tgt_slab + rdispl[d][s] .. + send_counts[s][d]*e) =
 *     input [s*in_slab  + sdispl[s][d] .. + send_counts[s][d]*e)
 *   with sdispl[s][d] = sum_{d'<d} send_counts[s][d']*e  (input packed by destination)
 *   and  rdispl[d][s] = sum_{s'<s} send_counts[s'][d]*e  (target packed by source)
 *   recv_counts[d][s] = send_counts[s][d]
 *   signal[r][b] += 1 for every rank r < P and admitted block b < B
 *
 * Counts scale by the type size as in the ncclx ctranAllToAllvIbImpl
 * pseudocode on the "vccl alltoallv dev log" page (section 5).  B is
 * CalAllToAllVBlocks(P, core_num) ("Launch width" section of the PyPTO page).
 * The create/run split mirrors the two-phase aclnn calling convention of the
 * CANN BatchMatMulReduceScatterAllToAll page (section "Two-phase API"), and
 * exchanges whose payload exceeds 1 GiB are issued as several launches of at
 * most 1 GiB each, after the chunk rule of the vccl page (section 2).
 *
 * All device pointers are plain device addresses (hipMalloc or torch CUDA
 * memory).  The library never allocates, copies or keeps payload buffers: it
 * owns only a small workspace allocated by a2av_create.
 *
 * Thread safety: a handle is not thread-safe and its workspace is shared by
 * all runs on it; runs on one handle must be ordered (one stream, or streams
 * the caller orders).  Use one handle per concurrent stream.
 *
 * Processes: a run with B > 1 ends in a cooperative launch.  On ROCm a
 * process that has made a cooperative launch keeps the device's resource for
 * them until it exits, and meanwhile another process's cooperative launch on
 * the same GPU fails (A2AV_ERR_HIP, "the operation cannot be performed in the
 * present state").  Runs with B = 1 are unaffected.  Drive each GPU from one
 * process.
 *
 * Graphs: a run enqueues only kernel launches on its stream (no copies, no
 * memsets, no synchronization), so a run may be captured into a HIP graph;
 * every replay is one more run over the buffers' contents at replay time,
 * ordered with the handle's other runs like any run.  A handle created with
 * A2AV_FLAG_PROFILE records no events while its stream is capturing.
 */
#ifndef A2AV_H
#define A2AV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct a2av_handle a2av_handle;

/* Payload element type.  a2av_run / a2av_run_blocked take FP32 and INT8 only
 * ("Constraints and diagnostics" section of the PyPTO page) and move raw
 * bits.  FP16 and BF16 are the payloads of a2av_run_bias, which adds. */
enum a2av_dtype { A2AV_FP32 = 0, A2AV_INT8 = 1, A2AV_FP16 = 2, A2AV_BF16 = 3 };

/* Status codes.  NULLPTR is kept apart from INVALID_ARGS as in the aclnn
 * error table (ACLNN_ERR_PARAM_NULLPTR vs ACLNN_ERR_PARAM_INVALID). */
enum a2av_status {
    A2AV_OK = 0,
    A2AV_ERR_NULLPTR = 1,           /* a required pointer is NULL               */
    A2AV_ERR_INVALID_ARGS = 2,      /* bad size, range, stride, alias or signal */
    A2AV_ERR_UNSUPPORTED_DTYPE = 3, /* dtype not one the entry point takes      */
    A2AV_ERR_OVER_CAPACITY = 4,     /* a row or column of counts overflows its slab */
    A2AV_ERR_LAUNCH_CAPACITY = 5,   /* B > 1 blocks cannot all be co-resident   */
    A2AV_ERR_HIP = 6,               /* a HIP runtime call failed                */
    A2AV_ERR_TIMEOUT = 7            /* the block barrier's bounded wait expired; the
                                       run's copies and flags still complete */
};

/* a2av_config.flags */
#define A2AV_FLAG_PROFILE 1u /* time each run: HIP events before and after K1 and
                                 after the last K2 launch */
/* With B > 1, make the final launch a regular one and skip the wait for the
 * other blocks.  Every admitted block still raises its own flags once its
 * copies are done, the co-resident capacity is still checked (B above it is
 * LAUNCH_CAPACITY), and the results, flags included, are those of the
 * cooperative run: on one GPU the wait is not observable, since the flags are
 * raised before it and the kernel's end already orders every copy before
 * later work on the stream.  What it saves is the cooperative launch's own
 * cost (about 20 us of idle GPU per run on an MI355X: the HIP runtime runs
 * cooperative launches on a second hardware queue, and the hand-offs to and
 * from it leave the GPU idle).  The default keeps the all-resident launch of
 * the "Launch width" section of the PyPTO page. */
#define A2AV_FLAG_NO_BLOCK_WAIT 2u

typedef struct a2av_config {
    int32_t device;            /* HIP device ordinal the handle binds to                 */
    int32_t P;                 /* virtual ranks, 1..64 (NR of the [NR, S] signal)        */
    int64_t in_slab_bytes;     /* byte stride between input slabs, >= 1                  */
    int64_t tgt_slab_bytes;    /* byte stride between target slabs, >= 1                 */
    int32_t S;                 /* signal row stride in int32 elements, >= 1              */
    int32_t wg_per_block;      /* workgroups per admitted block; 0 = chosen at create    */
    int64_t chunk_limit_bytes; /* payload bytes per K2 launch; 0 = 2^30 (1 GiB)          */
    int64_t capacity_override; /* co-resident workgroup limit; 0 = query the device      */
    uint32_t flags;            /* A2AV_FLAG_*                                            */
    int32_t spin_limit;        /* barrier poll limit; 0 = default (about 1 s)            */
} a2av_config;

/* What one a2av_run with a given core_num launches (for logs and benches). */
typedef struct a2av_launch_info {
    int64_t blocks;            /* B = CalAllToAllVBlocks(P, core_num)                    */
    int32_t wg_per_block;      /* G: workgroups that execute one admitted block          */
    int32_t workgroups;        /* W = B * G workgroups per K2 launch                     */
    int32_t threads_per_wg;    /* K2 workgroup size (the bias exchange's K2 runs 512)    */
    int32_t chunk_launches;    /* K2 launches per run (host chunk plan)                  */
    int64_t chunk_limit_bytes; /* payload bytes per K2 launch                            */
    int64_t capacity;          /* co-resident K2 workgroups on the device                */
    int32_t cooperative;       /* 1 when the last K2 launch is cooperative (B > 1)      */
    int32_t reserved;
} a2av_launch_info;

/*
 * Create a handle bound to cfg->device: checks the geometry (P in 1..64,
 * slabs >= 1, S >= 1, chunk limit >= 0 and at most 2^20 launches to cover
 * P * min(slabs) bytes), queries the co-resident capacity of
 * the copy kernel and allocates the workspace (displacement tables, plan
 * words, block counters, the latched error word).
 * Returns A2AV_OK and sets *out, or an error with *out left NULL.
 * Errors: NULLPTR (out or cfg NULL), INVALID_ARGS (geometry), HIP.
 */
int a2av_create(a2av_handle **out, const a2av_config *cfg);

/*
 * Enqueue one exchange on `stream` (a hipStream_t; NULL = default stream).
 *   input        device, P*in_slab bytes, read only
 *   target       device, P*tgt_slab bytes; only the received prefix of each
 *                slab is written, the rest keeps its bytes
 *   signal       device int32 [P, S], row-major; entries (r < P, b < B) +1
 *   send_counts  device int32 [P, P], row-major [s][d], element counts, read only
 *   recv_counts  device int32 [P, P], row-major [d][s], overwritten
 *   P            must equal the handle's P (the rank count is an explicit
 *                argument here, where the page's kernel reads it from its
 *                communication context)
 *   core_num     requested block limit L, 1..INT32_MAX
 *   dtype        A2AV_FP32 or A2AV_INT8
 *
 * Checked on the host before anything is enqueued, first failure wins:
 *   NULLPTR (any operand) -> UNSUPPORTED_DTYPE -> INVALID_ARGS (P differs
 *   from the handle, core_num out of range, S < B) -> LAUNCH_CAPACITY (B > 1
 *   and B above the co-resident capacity: refused, never partially launched)
 *   -> INVALID_ARGS (two operands share a byte; a slab size not a whole
 *   number of elements).
 * Checked on the device by the count kernel, in this order, before any
 * operand is written: a negative count (INVALID_ARGS), a source row or
 * destination column whose bytes exceed its slab (OVER_CAPACITY),
 * signal[r][b] (r < P, b < B) not all equal (INVALID_ARGS).  A device-side
 * failure writes nothing, is latched in the handle and is reported by
 * a2av_query_error; a2av_run itself has already returned A2AV_OK.
 * The call does not synchronize: results are visible to later work on
 * `stream`.  Returns A2AV_ERR_HIP if a launch fails.  recv_counts and the
 * signal are written only by the run's final launch, so a run of one copy
 * launch (payload up to the chunk limit) whose launch is refused writes
 * nothing, as "Launch width" asks of a refused start; in a run of several
 * chunk launches the chunks copied before the failing launch stay in the
 * target.
 */
int a2av_run(a2av_handle *h, const void *input, void *target, int32_t *signal,
             const int32_t *send_counts, int32_t *recv_counts, int32_t P, int64_t core_num,
             int32_t dtype, void *stream);

/*
 * The blocked exchange: a2av_run where each segment s -> d is read from the
 * source as nblk equal sub-blocks instead of one contiguous run.  Source slab
 * s is nblk block-rows of row_s/nblk bytes (row_s = the bytes s sends); each
 * block-row lists the sub-blocks for destinations 0..P-1 in order, sub-block
 * d being send_counts[s][d]/nblk elements.  The target is as in a2av_run:
 * segment s -> d lands at rdispl[d][s], its sub-blocks in block-row order.
 * This is the AllToAll at the end of the CANN
 * BatchMatMulReduceScatterAllToAll op taken on the source's own layout
 * ("Function and computation flow", "Constraints": per rank temp3 is
 * (E/ep, ep*C, H/tp), y is (E, C, H/tp)): with nblk = E/ep and every count
 * C*H/tp*nblk, block-row a is expert a's (ep*C, H/tp) slice, so the pack
 * into destination order that would precede a2av_run is fused away.
 * nblk = 1 is exactly a2av_run.
 * Errors: as a2av_run; in addition nblk < 1 is INVALID_ARGS (host, with the
 * P check), and a count that nblk does not divide is INVALID_ARGS on the
 * device (right after the negative-count check, latched like the others).
 */
int a2av_run_blocked(a2av_handle *h, const void *input, void *target, int32_t *signal,
                     const int32_t *send_counts, int32_t *recv_counts, int32_t P,
                     int64_t core_num, int32_t dtype, int32_t nblk, void *stream);

/*
 * The blocked exchange with the bias Add fused in front: the tail of the CANN
 * BatchMatMulReduceScatterAllToAll op ("Function and computation flow":
 * temp3 = temp2 + bias, y = AllToAll(temp3); "Parameters": BFLOAT16 x takes
 * an FP32 bias and adds in FP32, FLOAT16 x takes an FP16 bias; "Constraints",
 * yShardType 0: bias (E/ep, 1, H/tp) broadcast over the C rows).
 *   input   temp2 of every rank, as in a2av_run_blocked (nblk = E/ep
 *           block-rows per source), 16-bit elements (FP16 or BF16 bits)
 *   bias    device, [P, nblk, hidden] values: FP32 for BF16, FP16 for FP16;
 *           element h of a row in block-row a of source s gets
 *           bias[(s*nblk + a)*hidden + h]; read only
 *   hidden  elements per row (H/tp)
 * Every output element is the sum formed in FP32 and rounded once, to
 * nearest even, to the payload type; target, signal and recv_counts are as
 * in a2av_run_blocked.  Counts must be whole rows of every sub-block
 * (multiples of nblk * hidden; INVALID_ARGS on the device otherwise).
 * Host checks, first failure wins: NULLPTR (any of the six operands) ->
 * UNSUPPORTED_DTYPE (not FP16/BF16) -> INVALID_ARGS (P, nblk < 1, hidden < 1,
 * core_num, S < B) -> LAUNCH_CAPACITY -> INVALID_ARGS (two of the six
 * operands share a byte; a slab not a whole number of elements; and, as
 * limits of this implementation, hidden not a multiple of 8 or above 2^28,
 * or input, target, bias, slabs or the chunk limit not 16-byte aligned).
 */
int a2av_run_bias(a2av_handle *h, const void *input, void *target, int32_t *signal,
                  const int32_t *send_counts, int32_t *recv_counts, const void *bias, int32_t P,
                  int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden, void *stream);

/*
 * indexed_all_to_all_v: the six-operand variant named in the "A5 URMA indexed
 * exchange" section of the LowerL2TensorCollectives page (index the sixth
 * operand, local to the sender).  The page does not say what index means;
 * this library reads it as the sender's row gather list.
 *   input   P token tables at stride in_slab bytes; table s holds
 *           in_slab / (row_elems * e) whole rows of row_elems elements
 *   index   device, int32 [P, index_stride], read only: the rows source s
 *           sends, for d = 0..P-1 in turn, are table rows index[s][0],
 *           index[s][1], ...; a row may be named any number of times;
 *           entries past the rows a source sends are ignored (all
 *           P * index_stride entries must be allocated: the device may load
 *           them, but their values never affect the result)
 *   send_counts / recv_counts / target / signal as in a2av_run (counts in
 *           elements, whole rows)
 * Segment s -> d lands where a2av_run puts it: the exchange of the packed
 * rows, without packing them.
 * Host checks, first failure wins: NULLPTR (any of the six operands) ->
 * UNSUPPORTED_DTYPE (not FP32/INT8) -> INVALID_ARGS (P, row_elems < 1,
 * index_stride < 1, core_num, S < B) -> LAUNCH_CAPACITY -> INVALID_ARGS (two
 * of the six operands share a byte; a slab not a whole number of elements).
 * Device checks (a2av_query_error), nothing written on failure: a negative
 * count -> INVALID_ARGS; a count that is not whole rows -> INVALID_ARGS; a
 * source sending more rows than index_stride or a column over tgt_slab ->
 * OVER_CAPACITY; an index entry in use outside the table -> INVALID_ARGS;
 * unequal signal -> INVALID_ARGS.
 */
int a2av_run_indexed(a2av_handle *h, const void *input, void *target, int32_t *signal,
                     const int32_t *send_counts, int32_t *recv_counts, const int32_t *index,
                     int32_t P, int64_t core_num, int32_t dtype, int32_t row_elems,
                     int64_t index_stride, void *stream);

/*
 * a2av_run with a host copy of the counts, for callers that hold them on the
 * host (the counts computed on the host side and passed down, as in log C of
 * section 7 of the vccl alltoallv dev log).  Two things change:
 *   - the count checks run on the host, before anything is enqueued, and
 *     their status is the call's return value: a negative count
 *     (INVALID_ARGS), then a source row or destination column over its slab
 *     (OVER_CAPACITY), after the host checks of a2av_run and in the
 *     device's order;
 *   - the chunk plan follows the payload T: ceil(T / limit) launches (at
 *     least one) instead of enough to cover the geometry bound
 *     P * min(in_slab, tgt_slab) (section 2 of the same page re-enqueues by
 *     the op's bytes).
 *   host_send_counts  host int32 [P, P], row-major [s][d], read only; it
 *                     must hold the same counts as send_counts (device)
 * Everything else is a2av_run: the device still checks send_counts and the
 * signal (latched, a2av_query_error).  If the device counts differ from the
 * host copy and their payload exceeds what the planned launches cover, the
 * run is refused on the device with OVER_CAPACITY and writes nothing.
 */
int a2av_run_host_counts(a2av_handle *h, const void *input, void *target, int32_t *signal,
                         const int32_t *send_counts, int32_t *recv_counts,
                         const int32_t *host_send_counts, int32_t P, int64_t core_num,
                         int32_t dtype, void *stream);

/* The host part of a2av_run_host_counts alone (no GPU needed): the count
 * checks on `host_send_counts` for a handle created with `cfg` (cfg->P
 * ranks, its slabs, its chunk limit, 0 = 1 GiB) and elements of `dtype`
 * (FP32 or INT8).  Returns the status the call would return for the counts
 * and, on A2AV_OK, the payload in bytes and the number of chunk launches.
 * Errors: NULLPTR, UNSUPPORTED_DTYPE, INVALID_ARGS (cfg geometry; a negative
 * count), OVER_CAPACITY. */
int a2av_check_host_counts(const a2av_config *cfg, const int32_t *host_send_counts,
                           int32_t dtype, int64_t *payload_bytes, int32_t *launches);

/*
 * a2av_run_blocked, a2av_run_bias and a2av_run_indexed with a host copy of
 * the counts (the host-side counts of log C, section 7 of the vccl alltoallv
 * dev log), as a2av_run_host_counts is to a2av_run.  Each takes its
 * exchange's arguments and host_send_counts (host int32 [P, P], row-major
 * [s][d], read only, the same counts as send_counts on the device), runs that
 * exchange's host checks, then the count checks on the host copy in the
 * device's order, whose status the call returns before anything is enqueued:
 *   1. a negative count                                  -> INVALID_ARGS
 *   2. a count that is not whole sub-blocks (blocked: a multiple of nblk),
 *      whole bias rows (bias: of nblk * hidden) or whole gathered rows
 *      (indexed: of row_elems)                           -> INVALID_ARGS
 *   3. a source over its limit (blocked and bias: its row's bytes over
 *      in_slab; indexed: more rows than index_stride) or a destination
 *      column's bytes over tgt_slab                     -> OVER_CAPACITY
 * The chunk plan follows the payload T: ceil(T / limit) launches (at least
 * one).  The device still checks send_counts, the gather-list entries in use
 * (indexed) and the signal, latched for a2av_query_error, and refuses a
 * payload the planned launches cannot cover (OVER_CAPACITY, nothing
 * written).  NULLPTR when h or host_send_counts is NULL.
 */
int a2av_run_blocked_host_counts(a2av_handle *h, const void *input, void *target,
                                 int32_t *signal, const int32_t *send_counts,
                                 int32_t *recv_counts, const int32_t *host_send_counts,
                                 int32_t P, int64_t core_num, int32_t dtype, int32_t nblk,
                                 void *stream);
int a2av_run_bias_host_counts(a2av_handle *h, const void *input, void *target, int32_t *signal,
                              const int32_t *send_counts, int32_t *recv_counts,
                              const void *bias, const int32_t *host_send_counts, int32_t P,
                              int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden,
                              void *stream);
int a2av_run_indexed_host_counts(a2av_handle *h, const void *input, void *target,
                                 int32_t *signal, const int32_t *send_counts,
                                 int32_t *recv_counts, const int32_t *index,
                                 const int32_t *host_send_counts, int32_t P, int64_t core_num,
                                 int32_t dtype, int32_t row_elems, int64_t index_stride,
                                 void *stream);

/* The count checks of the *_host_counts entry points alone (no GPU needed),
 * for a handle created with `cfg`: elements of `dtype` (FP32, INT8, FP16 or
 * BF16), every count a multiple of `unit` (1 for the plain exchange, nblk,
 * nblk * hidden or row_elems), and with index_stride > 0 the indexed
 * exchange's row limit in place of in_slab.  Returns the status the run
 * would return for the counts and, on A2AV_OK, the payload in bytes and the
 * number of chunk launches (cfg's chunk limit, 0 = 1 GiB).  Errors: NULLPTR,
 * UNSUPPORTED_DTYPE, INVALID_ARGS (cfg geometry, unit < 1, index_stride < 0,
 * or a count check), OVER_CAPACITY. */
int a2av_check_host_counts_ex(const a2av_config *cfg, const int32_t *host_send_counts,
                              int32_t dtype, int64_t unit, int64_t index_stride,
                              int64_t *payload_bytes, int32_t *launches);

/*
 * a2av_run without a handle, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Nothing is allocated: the workspace is one array of 192 KiB per
 * device, held by the library until the process ends, whose address is
 * looked up on the first call on each device (the device current at the
 * call).  Operands, layout, the exchange and the host checks are those of
 * a2av_run with the handle's geometry passed in (in_slab_bytes,
 * tgt_slab_bytes, S) and the defaults of a2av_create (1 GiB per launch, the
 * device's co-resident capacity, workgroups per block chosen as there).
 *   status  device int32, written by the run: A2AV_OK, or the device-side
 *           failure a2av_query_error would report (INVALID_ARGS,
 *           OVER_CAPACITY, TIMEOUT); caller-owned, a sixth operand that may
 *           not overlap the others
 * Errors returned by the call: NULLPTR (status or an operand NULL), the host
 * checks of a2av_run, INVALID_ARGS when P is over 64 or the device's
 * capacity needs a workspace larger than the array, HIP.
 * Every call on a GPU uses that GPU's one array, and each run clears what
 * must start at zero: calls whose runs overlap on one GPU (other threads,
 * unordered streams) race and give undefined results; order them.
 */
int a2av_run_noalloc(const void *input, void *target, int32_t *signal,
                     const int32_t *send_counts, int32_t *recv_counts, int32_t *status,
                     int32_t P, int64_t in_slab_bytes, int64_t tgt_slab_bytes, int32_t S,
                     int64_t core_num, int32_t dtype, void *stream);

/* Free the workspace and the handle (synchronizes the device first).
 * NULL is accepted and ignored.  The end of the create/run/destroy life
 * cycle: the CANN BatchMatMulReduceScatterAllToAll page ("Full example",
 * step 4) frees the workspace memory once the two-phase calls are done and
 * the stream has been synchronized. */
int a2av_destroy(a2av_handle *h);

/* CalAllToAllVBlocks(P, L): L when L < P, else the largest multiple of P not
 * exceeding L ("Launch width" section of the PyPTO page).  -1 if P < 1 or L < 1.
 * Pure host function. */
int64_t a2av_blocks(int64_t P, int64_t L);

/* Host-side checks of a2av_run, as a pure host function that never touches
 * device memory (usable without a GPU).  cfg gives P, slabs and S; `capacity`
 * is the co-resident limit (<= 0: no limit); `P` is the run's argument.
 * Returns the status a2av_run would return before enqueuing anything. */
int a2av_check_args(const a2av_config *cfg, int64_t capacity, const void *input,
                    const void *target, const int32_t *signal, const int32_t *send_counts,
                    const int32_t *recv_counts, int32_t P, int64_t core_num, int32_t dtype);

/* The host-side checks of a2av_run_bias and a2av_run_indexed alone (no GPU
 * needed; nothing is dereferenced): the status either entry point would
 * return before enqueuing anything, for a handle created with `cfg` (its
 * chunk limit included, 0 = the default) whose co-resident capacity is
 * `capacity` (0 = no limit). */
int a2av_check_bias_args(const a2av_config *cfg, int64_t capacity, const void *input,
                         const void *target, const int32_t *signal, const int32_t *send_counts,
                         const int32_t *recv_counts, const void *bias, int32_t P,
                         int64_t core_num, int32_t dtype, int32_t nblk, int32_t hidden);
int a2av_check_indexed_args(const a2av_config *cfg, int64_t capacity, const void *input,
                            const void *target, const int32_t *signal,
                            const int32_t *send_counts, const int32_t *recv_counts,
                            const int32_t *index, int32_t P, int64_t core_num, int32_t dtype,
                            int32_t row_elems, int64_t index_stride);

/* Wait for the handle's last stream, then return and clear the latched
 * device-side status (A2AV_OK when every run since the last query was valid;
 * otherwise the first failure: INVALID_ARGS, OVER_CAPACITY or TIMEOUT).
 * The latch follows the runtime fallback of the PyPTO page ("Current
 * limitations"): checks that can only run once the operands exist latch an
 * INVALID_ARGS status at the first violation instead of failing the call
 * that submitted the work.  Here the count and signal checks run on the
 * device, so a2av_run returns before their outcome is known; a caller that
 * needs it synchronously calls this function after the run.  This is a
 * departure from checking the counts on the host before any write, made so
 * that a run needs no device-to-host read-back. */
int a2av_query_error(a2av_handle *h);

/* Fill *out with what a run of a2av_run, a2av_run_blocked or a2av_run_bias
 * with `core_num` would launch: the admitted blocks B (CalAllToAllVBlocks,
 * "Launch width" section of the PyPTO page, which also refuses a
 * sync-start launch beyond the co-resident capacity instead of launching
 * part of it), the workgroups that run them, and the chunk launches of at
 * most chunk_limit_bytes each (the re-enqueue above 1 GB of section 2 of the
 * vccl alltoallv dev log).  a2av_run_indexed plans its own: its payload is
 * bounded by the smaller of P target slabs and P gather lists of index_stride
 * rows each (a row may be named many times).  Errors: NULLPTR,
 * INVALID_ARGS (core_num out of range), LAUNCH_CAPACITY. */
int a2av_launch_info_get(a2av_handle *h, int64_t core_num, a2av_launch_info *out);

/* With A2AV_FLAG_PROFILE: wait for the runs recorded since the last read (at
 * most the last 256) and report, summed over them, the count kernel's time
 * and the K2 time (end of K1 to end of the last K2 launch, so the gaps between
 * a run's K2 launches are included) in microseconds, the number of K2
 * launches and the number of runs; then start a new tally.
 * Returns INVALID_ARGS when the handle was created without profiling. */
int a2av_profile_read(a2av_handle *h, double *k1_us, double *k2_us, int32_t *k2_launches,
                      int32_t *runs);

/* With A2AV_FLAG_PROFILE: record the events on one run in `every`, counting
 * runs as they are enqueued from this call on (the first run after the call
 * is recorded), so that a series of short runs is timed on a sample instead
 * of paying the events' own cost (a few microseconds each on the stream) on
 * every run.  every = 1, the default, records every run.  Errors: NULLPTR,
 * INVALID_ARGS (every < 1, or a handle created without profiling). */
int a2av_profile_sample(a2av_handle *h, int32_t every);

/* Human-readable name of a status code (static storage), in the spirit of
 * the aclnn error table on the CANN page ("Two-phase API": a named status
 * per failure class, NULLPTR apart from INVALID).  Unknown codes give
 * "A2AV_ERR_UNKNOWN". */
const char *a2av_status_string(int status);

/* Text of the last failing HIP call on this handle ("" if none). */
const char *a2av_last_hip_error(a2av_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* A2AV_H */
