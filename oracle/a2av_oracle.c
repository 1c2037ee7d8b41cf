/*
 * a2av_oracle.c -- plain CPU oracle for the variable-count all-to-all exchange.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, helper or
 * table with the HIP library; the only thing the two agree on is the numeric
 * value of each status code, because both report to the same callers.
 *
 * What it computes (the op of the PyPTO "LowerL2TensorCollectives Pass" page,
 * section "Behavior": all_to_all_v(input, target, signal, send_counts,
 * recv_counts, core_num)), with P virtual ranks laid out as slabs of one
 * allocation:
 *
 *   input   P slabs of in_slab bytes, slab s packed by destination d = 0..P-1
 *   target  P slabs of tgt_slab bytes, slab d packed by source s = 0..P-1
 *   signal  [P, S] int32
 *   send_counts [P, P] int32, element counts, send_counts[s][d] = s -> d
 *   recv_counts [P, P] int32, written: recv_counts[d][s] = send_counts[s][d]
 *
 * The segment addressing follows the ncclx ctranAllToAllvIbImpl pseudocode on
 * the "vccl alltoallv dev log" page (section 5, "ref / meta ncclx"): the send
 * buffer of peer d starts at sendbuff + sDispls[d] * typeSize, the receive
 * buffer of peer s at recvbuff + rDispls[s] * typeSize, and sendCounts[d] *
 * typeSize bytes move.  The displacements are the exclusive prefix sums of the
 * counts (no displacement operand exists in the five-operand statement).
 *
 * What pins each function is recorded at its definition.  The signal update
 * (arrive) is this implementation's reading of the barrier the pages
 * describe; it is pinned against an event model of that block and
 * sequence-counter barrier, written apart from this file.  The plain, blocked
 * and indexed exchanges move raw bytes; the fused-bias exchange adds in
 * binary32 and rounds to the 16-bit payload type under IEEE 754's rules,
 * infinities and NaNs included.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* Status values (same numbers as the library reports). */
#define OR_OK 0
#define OR_ERR_NULLPTR 1
#define OR_ERR_INVALID_ARGS 2
#define OR_ERR_UNSUPPORTED_DTYPE 3
#define OR_ERR_OVER_CAPACITY 4
#define OR_ERR_LAUNCH_CAPACITY 5

#define OR_DTYPE_FP32 0
#define OR_DTYPE_INT8 1
#define OR_DTYPE_FP16 2
#define OR_DTYPE_BF16 3

#define OR_MAX_P 64
#define OR_INT32_MAX 2147483647LL

/*
 * CalAllToAllVBlocks(P, L): the admitted block count.  "Launch width" section
 * of the LowerL2TensorCollectives page: B = L when L < P, otherwise the
 * largest multiple of P that does not exceed L.  Written as the definition
 * (search downward from L for the first multiple of P), not as a division.
 * Returns -1 when P < 1 or L < 1.
 * Pinned by: the page's printed case L=10, P=8 -> 8, the rule L<P -> L, and a
 * brute-force enumeration of multiples in the tests.
 */
int64_t a2av_oracle_blocks(int64_t P, int64_t L)
{
    if (P < 1 || L < 1)
        return -1;
    if (L < P)
        return L;
    for (int64_t m = L; m >= P; --m)
        if (m % P == 0)
            return m;
    return -1; /* unreachable: P itself is a multiple of P and P <= L */
}

static int64_t elem_size(int32_t dtype)
{
    return dtype == OR_DTYPE_FP32 ? 4 : dtype == OR_DTYPE_INT8 ? 1 : 2;
}

/* Half-open byte ranges [a, a+na) and [b, b+nb) share at least one byte. */
static int ranges_overlap(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb)
{
    if (na == 0 || nb == 0)
        return 0;
    return a < b + nb && b < a + na;
}

/*
 * The argument checks, in this order (the first failing one is reported and
 * nothing is written):
 *   1. a null operand                                   -> NULLPTR
 *   2. dtype not FP32 / INT8 ("Constraints and diagnostics": the supported
 *      dtypes)                                          -> UNSUPPORTED_DTYPE
 *   3. P outside [1, 64], S < 1, a slab size < 1        -> INVALID_ARGS
 *   4. core_num outside [1, INT32_MAX] (same section)   -> INVALID_ARGS
 *   5. signal stride S < B, B the folded block count    -> INVALID_ARGS
 *   6. B > 1 and B above the co-resident capacity (all admitted blocks must be
 *      resident at once; an over-capacity sync-start launch is refused, not
 *      partially launched; "Launch width")              -> LAUNCH_CAPACITY
 *      (capacity <= 0 means "no limit"; the GPU's limit is a device property)
 *   7. any two of the five operands share a byte (the pairwise-distinct window
 *      rule of "Current limitations")                   -> INVALID_ARGS
 *   8. a slab size that is not a whole number of elements -> INVALID_ARGS
 *   9. a negative count                                 -> INVALID_ARGS
 *  9b. a count that nblk (times the row length, with a bias) does not
 *      divide (blocked and fused-bias exchanges only)   -> INVALID_ARGS
 *  10. a source row or destination column whose bytes exceed its slab
 *                                                       -> OVER_CAPACITY
 *  11. signal[r][b] (r < P, b < B) not all equal        -> INVALID_ARGS
 * Checks 9-11 are this implementation's reading of the count-matrix cases
 * the page's system test names (0 / 1 / capacity / over-capacity / negative)
 * and of the barrier's need for a common starting value.
 */
static int check_args(const void *input, const void *target, const int32_t *signal,
                      const int32_t *send_counts, const int32_t *recv_counts,
                      int32_t P, int32_t S, int64_t in_slab, int64_t tgt_slab,
                      int64_t core_num, int32_t dtype, int64_t capacity, int32_t nblk,
                      const void *bias, int32_t hidden)
{
    /* bias != NULL selects the fused-bias exchange: 16-bit payloads and a
     * sixth operand of P*nblk*hidden bias values. */
    const int with_bias = bias != NULL;
    if (!input || !target || !signal || !send_counts || !recv_counts)
        return OR_ERR_NULLPTR;
    if (with_bias ? (dtype != OR_DTYPE_FP16 && dtype != OR_DTYPE_BF16)
                  : (dtype != OR_DTYPE_FP32 && dtype != OR_DTYPE_INT8))
        return OR_ERR_UNSUPPORTED_DTYPE;
    if (P < 1 || P > OR_MAX_P || S < 1 || in_slab < 1 || tgt_slab < 1 || nblk < 1 || hidden < 1)
        return OR_ERR_INVALID_ARGS;
    if (core_num < 1 || core_num > OR_INT32_MAX)
        return OR_ERR_INVALID_ARGS;
    int64_t B = a2av_oracle_blocks(P, core_num);
    if ((int64_t)S < B)
        return OR_ERR_INVALID_ARGS;
    if (B > 1 && capacity > 0 && B > capacity)
        return OR_ERR_LAUNCH_CAPACITY;

    int64_t bias_e = dtype == OR_DTYPE_BF16 ? 4 : 2;
    uintptr_t base[6] = {(uintptr_t)input, (uintptr_t)target, (uintptr_t)signal,
                         (uintptr_t)send_counts, (uintptr_t)recv_counts, (uintptr_t)bias};
    uint64_t len[6] = {(uint64_t)P * (uint64_t)in_slab, (uint64_t)P * (uint64_t)tgt_slab,
                       (uint64_t)P * (uint64_t)S * 4u, (uint64_t)P * (uint64_t)P * 4u,
                       (uint64_t)P * (uint64_t)P * 4u,
                       with_bias ? (uint64_t)P * (uint64_t)nblk * (uint64_t)hidden * (uint64_t)bias_e
                                 : 0u};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (ranges_overlap(base[i], len[i], base[j], len[j]))
                return OR_ERR_INVALID_ARGS;

    int64_t e = elem_size(dtype);
    if (in_slab % e != 0 || tgt_slab % e != 0)
        return OR_ERR_INVALID_ARGS;

    for (int32_t s = 0; s < P; ++s)
        for (int32_t d = 0; d < P; ++d)
            if (send_counts[s * P + d] < 0)
                return OR_ERR_INVALID_ARGS;
    int64_t unit = (int64_t)nblk * hidden;
    for (int32_t s = 0; s < P; ++s)
        for (int32_t d = 0; d < P; ++d)
            if (send_counts[s * P + d] % unit != 0)
                return OR_ERR_INVALID_ARGS;

    for (int32_t s = 0; s < P; ++s) {
        int64_t row = 0;
        for (int32_t d = 0; d < P; ++d)
            row += (int64_t)send_counts[s * P + d];
        if (row * e > in_slab)
            return OR_ERR_OVER_CAPACITY;
    }
    for (int32_t d = 0; d < P; ++d) {
        int64_t col = 0;
        for (int32_t s = 0; s < P; ++s)
            col += (int64_t)send_counts[s * P + d];
        if (col * e > tgt_slab)
            return OR_ERR_OVER_CAPACITY;
    }

    int32_t first = signal[0];
    for (int32_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b)
            if (signal[(int64_t)r * S + b] != first)
                return OR_ERR_INVALID_ARGS;
    return OR_OK;
}

/* Argument checks alone (used by the tests to pin each diagnostic). */
int a2av_oracle_check(const void *input, const void *target, const int32_t *signal,
                      const int32_t *send_counts, const int32_t *recv_counts,
                      int32_t P, int32_t S, int64_t in_slab, int64_t tgt_slab,
                      int64_t core_num, int32_t dtype, int64_t capacity)
{
    return check_args(input, target, signal, send_counts, recv_counts, P, S, in_slab,
                      tgt_slab, core_num, dtype, capacity, 1, NULL, 1);
}

/*
 * Step 2: recv_counts[d][s] = send_counts[s][d].  Each destination learns how
 * much every source sends it: the count matrix transposed.
 * Pinned by: closed form (numpy transpose) in the tests.
 */
static void transpose_counts(const int32_t *send_counts, int32_t *recv_counts, int32_t P)
{
    for (int32_t s = 0; s < P; ++s)
        for (int32_t d = 0; d < P; ++d)
            recv_counts[d * P + s] = send_counts[s * P + d];
}

/*
 * Step 3: byte displacements, the exclusive prefix sums of the counts.
 *   sdispl[s][d] = sum over d' < d of send_counts[s][d'] * e  (send side)
 *   rdispl[d][s] = sum over s' < s of send_counts[s'][d] * e  (receive side)
 * Pinned by: closed form (numpy exclusive cumsum) in the tests.
 */
static void displacements(const int32_t *C, int32_t P, int64_t e,
                          int64_t *sdispl, int64_t *rdispl)
{
    for (int32_t s = 0; s < P; ++s) {
        int64_t off = 0;
        for (int32_t d = 0; d < P; ++d) {
            sdispl[s * P + d] = off;
            off += (int64_t)C[s * P + d] * e;
        }
    }
    for (int32_t d = 0; d < P; ++d) {
        int64_t off = 0;
        for (int32_t s = 0; s < P; ++s) {
            rdispl[d * P + s] = off;
            off += (int64_t)C[s * P + d] * e;
        }
    }
}

/*
 * Step 4, the payload move, one memcpy per (source, destination) segment:
 *   target[d*tgt_slab + rdispl[d][s] .. + C[s][d]*e) =
 *   input [s*in_slab  + sdispl[s][d] .. + C[s][d]*e)
 * Bytes of a target slab past its received total are left as they were.
 * Pinned by: brute force (per-slab byte concatenation) on every count matrix
 * in {0,1,2}^(2x2) and {0,1}^(3x3), the P=1 identity, the equal-count case
 * reducing to a block transpose, and the round trip with transposed counts.
 */
static void move_segments(const uint8_t *input, uint8_t *target, const int32_t *C,
                          int32_t P, int64_t e, int64_t in_slab, int64_t tgt_slab,
                          const int64_t *sdispl, const int64_t *rdispl)
{
    for (int32_t s = 0; s < P; ++s)
        for (int32_t d = 0; d < P; ++d) {
            int64_t nbytes = (int64_t)C[s * P + d] * e;
            if (nbytes == 0)
                continue;
            memcpy(target + (int64_t)d * tgt_slab + rdispl[d * P + s],
                   input + (int64_t)s * in_slab + sdispl[s * P + d], (size_t)nbytes);
        }
}

/*
 * Step 5, the signal: every block b < B of every rank r < P arrives once, so
 * signal[r][b] grows by one (32-bit wraparound); entries with b >= B are left
 * alone.  The pages fix only that the signal is [NR, S] with S >= B and that
 * reusing it orders exchanges; the +1-per-exchange value is this
 * implementation's reading of the per-peer sequence-counter barrier on the
 * "vccl alltoallv dev log" page (section 6.1) and the block-aware barrier of
 * the LowerL2TensorCollectives page ("Launch width").
 * Pinned by: an event model of that barrier (every admitted block of every
 * rank posts its own wrapping counter once and waits for all to move past
 * the common entry value, in random interleavings), over random P, S and B,
 * entry values at the int32 edges and sequences of exchanges whose block
 * count changes; the model also decides which exchanges are refused.
 */
static void arrive(int32_t *signal, int32_t P, int32_t S, int64_t B)
{
    for (int32_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b) {
            uint32_t v = (uint32_t)signal[(int64_t)r * S + b];
            signal[(int64_t)r * S + b] = (int32_t)(v + 1u);
        }
}

/*
 * The whole exchange on host buffers.  Returns a status; on any error no
 * output byte changes.  capacity <= 0 disables the co-resident check.
 */
int a2av_oracle_run(const void *input, void *target, int32_t *signal,
                    const int32_t *send_counts, int32_t *recv_counts,
                    int32_t P, int32_t S, int64_t in_slab, int64_t tgt_slab,
                    int64_t core_num, int32_t dtype, int64_t capacity)
{
    int st = check_args(input, target, signal, send_counts, recv_counts, P, S, in_slab,
                        tgt_slab, core_num, dtype, capacity, 1, NULL, 1);
    if (st != OR_OK)
        return st;
    int64_t e = elem_size(dtype);
    int64_t B = a2av_oracle_blocks(P, core_num);
    int64_t sdispl[OR_MAX_P * OR_MAX_P];
    int64_t rdispl[OR_MAX_P * OR_MAX_P];
    transpose_counts(send_counts, recv_counts, P);
    displacements(send_counts, P, e, sdispl, rdispl);
    move_segments((const uint8_t *)input, (uint8_t *)target, send_counts, P, e, in_slab,
                  tgt_slab, sdispl, rdispl);
    arrive(signal, P, S, B);
    return OR_OK;
}

/*
 * The blocked exchange: the AllToAll at the end of the CANN
 * BatchMatMulReduceScatterAllToAll op ("Function and computation flow",
 * "Constraints": per rank temp3 is (E/ep, ep*C, H/tp) and y is (E, C, H/tp)),
 * taken on the source's own layout instead of after a pack into
 * destination order.  Source slab s is nblk block-rows; block-row a holds,
 * for d = 0..P-1 in order, the a-th of the nblk equal sub-blocks of the
 * segment s -> d (send_counts[s][d] / nblk elements each).  Destination
 * slab d receives segment s -> d at rdispl[d][s] as before, its sub-blocks
 * in order a = 0..nblk-1:
 *   target[d*tgt_slab + rdispl[d][s] + a*sub .. + sub) =
 *   input [s*in_slab + a*row_s/nblk + sdispl[s][d]/nblk .. + sub)
 * with sub = send_counts[s][d]*e/nblk and row_s the bytes source s sends.
 * With E/ep experts per rank, ep ranks, C tokens per expert and H/tp
 * hidden: nblk = E/ep and every count is C*H/tp*nblk, so block-row a is
 * expert a's (ep*C, H/tp) slice and sub-block d of it is rows d*C..d*C+C.
 * nblk = 1 is the plain exchange.  nblk < 1 is INVALID_ARGS among the
 * geometry checks; a count that nblk does not divide is INVALID_ARGS right
 * after the negative-count check (check 9b).
 * Pinned by: nblk = 1 equals a2av_oracle_run; the CANN layout relation
 * checked against numpy's transpose of (P, A, P, Q) to (P, P, A, Q); brute
 * force for tiny P in the tests.
 */
int a2av_oracle_run_blocked(const void *input, void *target, int32_t *signal,
                            const int32_t *send_counts, int32_t *recv_counts, int32_t P,
                            int32_t S, int64_t in_slab, int64_t tgt_slab, int64_t core_num,
                            int32_t dtype, int64_t capacity, int32_t nblk)
{
    int st = check_args(input, target, signal, send_counts, recv_counts, P, S, in_slab,
                        tgt_slab, core_num, dtype, capacity, nblk, NULL, 1);
    if (st != OR_OK)
        return st;

    int64_t e = elem_size(dtype);
    int64_t B = a2av_oracle_blocks(P, core_num);
    int64_t sdispl[OR_MAX_P * OR_MAX_P];
    int64_t rdispl[OR_MAX_P * OR_MAX_P];
    transpose_counts(send_counts, recv_counts, P);
    displacements(send_counts, P, e, sdispl, rdispl);
    for (int32_t s = 0; s < P; ++s) {
        int64_t row = 0;
        for (int32_t d = 0; d < P; ++d)
            row += (int64_t)send_counts[s * P + d] * e;
        for (int32_t d = 0; d < P; ++d) {
            int64_t sub = (int64_t)send_counts[s * P + d] * e / nblk;
            if (sub == 0)
                continue;
            for (int32_t a = 0; a < nblk; ++a)
                memcpy((uint8_t *)target + (int64_t)d * tgt_slab + rdispl[d * P + s] + a * sub,
                       (const uint8_t *)input + (int64_t)s * in_slab + a * (row / nblk) +
                           sdispl[s * P + d] / nblk,
                       (size_t)sub);
        }
    }
    arrive(signal, P, S, B);
    return OR_OK;
}

/* ------------------------------------------------------------ 16-bit payload */

/* IEEE binary32 bits <-> float without aliasing tricks. */
static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/*
 * The 16-bit formats, from IEEE 754-2008 (binary16: 1 sign, 5 exponent and
 * 10 fraction bits, bias 15) and the bfloat16 layout (the upper half of a
 * binary32: 1 sign, 8 exponent and 7 fraction bits, bias 127).  Every
 * conversion takes and returns bit patterns, so NaN payloads cross the
 * boundary untouched.
 *
 * Narrowing (binary32 -> 16 bits) rounds to nearest, ties to even, the
 * default rounding of IEEE 754 (section 4.3.1):
 *   - a finite value is scaled into the grid of its binade (the subnormal
 *     grid below the format's smallest normal binade), the scaled value is
 *     rounded to an integer with ties to even, and the fields are assembled;
 *     a result at or past the largest finite value's next binade is an
 *     overflow, which under this rounding gives the infinity of the sign
 *     (section 7.4);
 *   - an infinity stays the infinity of the same sign;
 *   - a NaN becomes a quiet NaN (section 6.2): the sign and the leading
 *     payload bits are kept and the quiet bit is set.  IEEE 754 does not fix
 *     which NaN an operation returns, so the tests compare NaN-ness only.
 * Widening (16 bits -> binary32) is exact for every input: subnormals become
 * normals, infinities stay infinities, and a NaN keeps its sign and payload.
 */

/* bfloat16 -> binary32: the bits move to the upper half (exact, NaN payload
 * kept).  Pinned by: torch's CPU bfloat16 -> float32 on all 65,536 patterns. */
uint32_t a2av_oracle_bf16_to_f32(uint16_t h)
{
    return (uint32_t)h << 16;
}

/* Round the non-negative finite value a to nearest, ties to even, in a format
 * with `sig` significand bits (implicit bit included) whose smallest normal
 * binade is 2^emin; e is a's binade from its binary32 exponent field.  Returns
 * the rounded significand m (in [0, 2^sig]) and sets *binade to the binade
 * of its grid (emin for the subnormal grid). */
static int64_t round_to_grid(double a, int e, int emin, int sig, int *binade)
{
    if (e < emin)
        e = emin;                                      /* subnormal grid */
    double step = ldexp(1.0, e - (sig - 1));           /* one ulp in binade e */
    double q = a / step;                               /* exact: a power-of-2 scale */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0))
        r += 1.0;
    *binade = e;
    return (int64_t)r;
}

/* binary32 -> bfloat16, round to nearest, ties to even, as stated above.
 * Pinned by: torch's CPU float32 -> bfloat16 conversion on random bit
 * patterns of every exponent, ties, subnormals, the overflow edge, the
 * infinities and NaNs (NaN-ness only). */
uint16_t a2av_oracle_f32_to_bf16(uint32_t u)
{
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t efield = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (efield == 0xFFu) {
        if (frac == 0)
            return (uint16_t)(sign | 0x7F80u);                      /* +-Inf */
        return (uint16_t)(sign | 0x7FC0u | (uint16_t)(frac >> 16)); /* quiet NaN */
    }
    double a = fabs((double)f32_from_bits(u));
    if (a == 0.0)
        return sign;
    int binade;
    int64_t m = round_to_grid(a, (int)efield - 127, -126, 8, &binade);
    int64_t biased = (int64_t)binade + 127;
    if (m >= 256) {                                    /* rounded into the next binade */
        m >>= 1;
        biased += 1;
    }
    if (biased >= 255)                                 /* overflow */
        return (uint16_t)(sign | 0x7F80u);
    if (m < 128)                                       /* subnormal (or zero) result */
        return (uint16_t)(sign | (uint16_t)m);
    return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)(m & 0x7F));
}

/* binary16 -> binary32, exact.  Pinned by: numpy's float16 -> float32 on all
 * 65,536 patterns (NaN-ness only for NaNs). */
uint32_t a2av_oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t exp = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t man = (uint32_t)h & 0x3FFu;
    if (exp == 0x1Fu)                                  /* +-Inf, or NaN with its payload */
        return (sign << 31) | 0x7F800000u | (man << 13);
    float mag;
    if (exp == 0)
        mag = (float)man * (1.0f / 16777216.0f);       /* man * 2^-24, exact */
    else
        mag = f32_from_bits(((exp + 112u) << 23) | (man << 13)); /* rebias 15 -> 127 */
    return bits_from_f32(sign ? -mag : mag);
}

/* binary32 -> binary16, round to nearest, ties to even, as stated above.
 * Pinned by: numpy's float32 -> float16 conversion on random bit patterns of
 * every exponent, ties in the normal and subnormal ranges, the overflow edge
 * (65504, 65519, 65520, 70000, 131008), the infinities and NaNs (NaN-ness
 * only). */
uint16_t a2av_oracle_f32_to_f16(uint32_t u)
{
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t efield = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (efield == 0xFFu) {
        if (frac == 0)
            return (uint16_t)(sign | 0x7C00u);                      /* +-Inf */
        return (uint16_t)(sign | 0x7E00u | (uint16_t)(frac >> 13)); /* quiet NaN */
    }
    double a = fabs((double)f32_from_bits(u));
    if (a == 0.0)
        return sign;
    int binade;
    int64_t m = round_to_grid(a, (int)efield - 127, -14, 11, &binade);
    int64_t biased = (int64_t)binade + 15;
    if (m >= 2048) {                                   /* rounded into the next binade */
        m >>= 1;
        biased += 1;
    }
    if (biased >= 31)                                  /* overflow */
        return (uint16_t)(sign | 0x7C00u);
    if (m < 1024)                                      /* subnormal (or zero) result */
        return (uint16_t)(sign | (uint16_t)m);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)(m & 0x3FF));
}

/*
 * The exchange with the bias Add fused in front of it: the tail of the CANN
 * BatchMatMulReduceScatterAllToAll op ("Function and computation flow":
 * temp3 = temp2 + bias, y = AllToAll(temp3); "Parameters": for FLOAT16 x the
 * bias is FLOAT16, for BFLOAT16 x it is FLOAT32 and the add is done in FP32
 * and cast back; "Constraints", yShardType 0: bias (E/ep, 1, H/tp) broadcast
 * over the C rows).  Layout as in a2av_oracle_run_blocked with nblk = E/ep:
 * source s's block-row a is expert a; every element belongs to a row of
 * `hidden` (= H/tp) elements; element h of a row in block-row a of source s
 * gets bias[(s * nblk + a) * hidden + h].  Each sum is formed in binary32
 * (the FLOAT16 case widened the same way, a reading) and rounded once, to
 * nearest even, back to 16 bits.  Every IEEE class is taken as IEEE 754
 * gives it: a sum past the format's largest finite value is an infinity,
 * inf + (-inf) and any NaN operand give a NaN, subnormals add exactly.
 * The checks are check_args's with: bias a sixth operand (NULLPTR when
 * missing, in the pairwise-distinct rule with P*nblk*hidden values), dtype
 * FP16 or BF16 only, hidden >= 1 with the geometry, and every count a
 * multiple of hidden * nblk (whole rows of every sub-block; check 9b).
 * Pinned by: the conversion pins above; a zero bias reduces it to the
 * blocked exchange; the CANN layout relation against numpy / torch adds, on
 * moderate values and on values of every IEEE class (NaN-ness compared where
 * the result is a NaN).
 */
int a2av_oracle_run_bias(const void *input, void *target, int32_t *signal,
                         const int32_t *send_counts, int32_t *recv_counts, int32_t P, int32_t S,
                         int64_t in_slab, int64_t tgt_slab, int64_t core_num, int32_t dtype,
                         int64_t capacity, int32_t nblk, const void *bias, int32_t hidden)
{
    if (!bias)
        return OR_ERR_NULLPTR;
    int st = check_args(input, target, signal, send_counts, recv_counts, P, S, in_slab,
                        tgt_slab, core_num, dtype, capacity, nblk, bias, hidden);
    if (st != OR_OK)
        return st;

    int64_t B = a2av_oracle_blocks(P, core_num);
    int64_t sdispl[OR_MAX_P * OR_MAX_P];
    int64_t rdispl[OR_MAX_P * OR_MAX_P];
    transpose_counts(send_counts, recv_counts, P);
    displacements(send_counts, P, 2, sdispl, rdispl);
    const uint16_t *x = (const uint16_t *)input;
    uint16_t *y = (uint16_t *)target;
    for (int32_t s = 0; s < P; ++s) {
        int64_t row = 0; /* bytes source s sends */
        for (int32_t d = 0; d < P; ++d)
            row += (int64_t)send_counts[s * P + d] * 2;
        for (int32_t d = 0; d < P; ++d) {
            int64_t sub = (int64_t)send_counts[s * P + d] / nblk; /* elements */
            for (int32_t a = 0; a < nblk; ++a) {
                int64_t src = ((int64_t)s * in_slab + a * (row / nblk) + sdispl[s * P + d] / nblk) / 2;
                int64_t dst = ((int64_t)d * tgt_slab + rdispl[d * P + s]) / 2 + a * sub;
                for (int64_t k = 0; k < sub; ++k) {
                    int64_t h = k % hidden;
                    int64_t bi = ((int64_t)s * nblk + a) * hidden + h;
                    float sum;
                    if (dtype == OR_DTYPE_BF16) {
                        sum = f32_from_bits(a2av_oracle_bf16_to_f32(x[src + k])) +
                              ((const float *)bias)[bi];
                        y[dst + k] = a2av_oracle_f32_to_bf16(bits_from_f32(sum));
                    } else {
                        sum = f32_from_bits(a2av_oracle_f16_to_f32(x[src + k])) +
                              f32_from_bits(a2av_oracle_f16_to_f32(((const uint16_t *)bias)[bi]));
                        y[dst + k] = a2av_oracle_f32_to_f16(bits_from_f32(sum));
                    }
                }
            }
        }
    }
    arrive(signal, P, S, B);
    return OR_OK;
}

/* ------------------------------------------------------------ indexed exchange */

/*
 * indexed_all_to_all_v(input, target, signal, send_counts, recv_counts, index,
 * core_num): the variant named in the "A5 URMA indexed exchange" section of
 * the LowerL2TensorCollectives page, which gives its six operands (index the
 * sixth; input and index local to the sender, send_counts visible to peers)
 * but not what index means.  Reading taken here: index is the sender's row
 * gather list.  Input slab s is a table of rows of row_elems elements
 * (row_bytes = row_elems * e; the table holds in_slab / row_bytes rows); the
 * rows source s sends, in destination order d = 0..P-1 as in the plain
 * exchange, are the table rows named by index[s][0], index[s][1], ...  Row j
 * of segment s -> d is table row index[s][R(s,d) + j], R(s,d) the rows s
 * sends to destinations below d.  Target and signal are as in the plain
 * exchange: segment s -> d lands at rdispl[d][s] of slab d.  index is P
 * slabs of index_stride int32 entries; the same row may be named any number
 * of times.  This is the dispatch of an MoE layer with the pack folded in:
 * a token routed to two ranks is stored once and named twice.
 * Checks, first failure wins, nothing written on failure:
 *   1. a null operand (six)                             -> NULLPTR
 *   2. dtype not FP32 / INT8                            -> UNSUPPORTED_DTYPE
 *   3. P outside [1, 64], S < 1, a slab size < 1, row_elems < 1,
 *      index_stride < 1                                 -> INVALID_ARGS
 *   4-6. core_num range, S < B, launch capacity, as in check_args
 *   7. two of the six operands share a byte (index covers P*index_stride
 *      int32)                                           -> INVALID_ARGS
 *   8. a slab size that is not a whole number of elements -> INVALID_ARGS
 *   9. a negative count                                 -> INVALID_ARGS
 *  9b. a count that is not whole rows (row_elems does not divide it)
 *                                                       -> INVALID_ARGS
 *  10. a source that sends more rows than index_stride, or a destination
 *      column whose bytes exceed tgt_slab               -> OVER_CAPACITY
 * 10b. an index entry in use outside [0, in_slab / row_bytes)
 *                                                       -> INVALID_ARGS
 *  11. signal[r][b] (r < P, b < B) not all equal        -> INVALID_ARGS
 * Pinned by: index[s][k] = k on a packed input is the plain exchange; numpy
 * row gathers followed by the brute-force exchange; the MoE dispatch of
 * token tables equal to the plain exchange of the packed (duplicated)
 * tokens; every diagnostic in the tests.
 */
static int check_indexed(const void *input, const void *target, const int32_t *signal,
                         const int32_t *send_counts, const int32_t *recv_counts,
                         const int32_t *index, int32_t P, int32_t S, int64_t in_slab,
                         int64_t tgt_slab, int64_t core_num, int32_t dtype, int64_t capacity,
                         int32_t row_elems, int64_t index_stride)
{
    if (!input || !target || !signal || !send_counts || !recv_counts || !index)
        return OR_ERR_NULLPTR;
    if (dtype != OR_DTYPE_FP32 && dtype != OR_DTYPE_INT8)
        return OR_ERR_UNSUPPORTED_DTYPE;
    if (P < 1 || P > OR_MAX_P || S < 1 || in_slab < 1 || tgt_slab < 1 || row_elems < 1 ||
        index_stride < 1)
        return OR_ERR_INVALID_ARGS;
    if (core_num < 1 || core_num > OR_INT32_MAX)
        return OR_ERR_INVALID_ARGS;
    int64_t B = a2av_oracle_blocks(P, core_num);
    if ((int64_t)S < B)
        return OR_ERR_INVALID_ARGS;
    if (B > 1 && capacity > 0 && B > capacity)
        return OR_ERR_LAUNCH_CAPACITY;

    uintptr_t base[6] = {(uintptr_t)input, (uintptr_t)target, (uintptr_t)signal,
                         (uintptr_t)send_counts, (uintptr_t)recv_counts, (uintptr_t)index};
    uint64_t len[6] = {(uint64_t)P * (uint64_t)in_slab, (uint64_t)P * (uint64_t)tgt_slab,
                       (uint64_t)P * (uint64_t)S * 4u, (uint64_t)P * (uint64_t)P * 4u,
                       (uint64_t)P * (uint64_t)P * 4u, (uint64_t)P * (uint64_t)index_stride * 4u};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (ranges_overlap(base[i], len[i], base[j], len[j]))
                return OR_ERR_INVALID_ARGS;

    int64_t e = elem_size(dtype);
    if (in_slab % e != 0 || tgt_slab % e != 0)
        return OR_ERR_INVALID_ARGS;

    for (int32_t i = 0; i < P * P; ++i)
        if (send_counts[i] < 0)
            return OR_ERR_INVALID_ARGS;
    for (int32_t i = 0; i < P * P; ++i)
        if (send_counts[i] % row_elems != 0)
            return OR_ERR_INVALID_ARGS;

    for (int32_t s = 0; s < P; ++s) {
        int64_t rows = 0;
        for (int32_t d = 0; d < P; ++d)
            rows += send_counts[s * P + d] / row_elems;
        if (rows > index_stride)
            return OR_ERR_OVER_CAPACITY;
    }
    for (int32_t d = 0; d < P; ++d) {
        int64_t col = 0;
        for (int32_t s = 0; s < P; ++s)
            col += (int64_t)send_counts[s * P + d];
        if (col * e > tgt_slab)
            return OR_ERR_OVER_CAPACITY;
    }

    int64_t table_rows = in_slab / (row_elems * e);
    for (int32_t s = 0; s < P; ++s) {
        int64_t rows = 0;
        for (int32_t d = 0; d < P; ++d)
            rows += send_counts[s * P + d] / row_elems;
        for (int64_t k = 0; k < rows; ++k) {
            int32_t v = index[(int64_t)s * index_stride + k];
            if (v < 0 || (int64_t)v >= table_rows)
                return OR_ERR_INVALID_ARGS;
        }
    }

    int32_t first = signal[0];
    for (int32_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b)
            if (signal[(int64_t)r * S + b] != first)
                return OR_ERR_INVALID_ARGS;
    return OR_OK;
}

int a2av_oracle_run_indexed(const void *input, void *target, int32_t *signal,
                            const int32_t *send_counts, int32_t *recv_counts,
                            const int32_t *index, int32_t P, int32_t S, int64_t in_slab,
                            int64_t tgt_slab, int64_t core_num, int32_t dtype, int64_t capacity,
                            int32_t row_elems, int64_t index_stride)
{
    int st = check_indexed(input, target, signal, send_counts, recv_counts, index, P, S,
                           in_slab, tgt_slab, core_num, dtype, capacity, row_elems, index_stride);
    if (st != OR_OK)
        return st;

    int64_t e = elem_size(dtype);
    int64_t row_bytes = row_elems * e;
    int64_t B = a2av_oracle_blocks(P, core_num);
    int64_t sdispl[OR_MAX_P * OR_MAX_P];
    int64_t rdispl[OR_MAX_P * OR_MAX_P];
    transpose_counts(send_counts, recv_counts, P);
    displacements(send_counts, P, e, sdispl, rdispl);
    for (int32_t s = 0; s < P; ++s) {
        const uint8_t *table = (const uint8_t *)input + (int64_t)s * in_slab;
        const int32_t *list = index + (int64_t)s * index_stride;
        int64_t k = 0; /* position in source s's gather list */
        for (int32_t d = 0; d < P; ++d) {
            int64_t rows = send_counts[s * P + d] / row_elems;
            uint8_t *seg = (uint8_t *)target + (int64_t)d * tgt_slab + rdispl[d * P + s];
            for (int64_t j = 0; j < rows; ++j, ++k)
                memcpy(seg + j * row_bytes, table + (int64_t)list[k] * row_bytes,
                       (size_t)row_bytes);
        }
    }
    arrive(signal, P, S, B);
    return OR_OK;
}

/* Displacements alone, for the closed-form pins (no checks). */
void a2av_oracle_displacements(const int32_t *send_counts, int32_t P, int32_t dtype,
                               int64_t *sdispl, int64_t *rdispl)
{
    displacements(send_counts, P, elem_size(dtype), sdispl, rdispl);
}

/*
 * The segment-copy step alone on prepared buffers (no checks, counts assumed
 * valid): the loop the benchmark times as the CPU baseline.
 */
void a2av_oracle_move(const void *input, void *target, const int32_t *send_counts,
                      int32_t P, int32_t dtype, int64_t in_slab, int64_t tgt_slab)
{
    int64_t e = elem_size(dtype);
    int64_t sdispl[OR_MAX_P * OR_MAX_P];
    int64_t rdispl[OR_MAX_P * OR_MAX_P];
    displacements(send_counts, P, e, sdispl, rdispl);
    move_segments((const uint8_t *)input, (uint8_t *)target, send_counts, P, e, in_slab,
                  tgt_slab, sdispl, rdispl);
}
