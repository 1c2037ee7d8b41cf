/*
 * a2av_c_driver.c -- test program: the library's C ABI driven from C alone.
 *
 * For a few seeded exchanges (plain FP32 and INT8, chunked, blocked, BF16 and
 * FP16 with the bias Add, indexed, the plain exchange with a host copy of the
 * counts, and the entry point that allocates nothing)
 * it allocates the five operands with hipMalloc, calls a2av_create, two runs
 * of the entry point on a stream of its own, a2av_query_error and
 * a2av_destroy, then runs the CPU oracle twice on host copies of the same
 * inputs and compares the whole target allocation, the signal and
 * recv_counts byte for byte.  Test infrastructure: it links the oracle.
 * Exit status 0 when every case matches, 1 on a mismatch, 2 on a HIP or
 * library error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "a2av.h"

/* The oracle's entry points (oracle/a2av_oracle.c, which has no header). */
int a2av_oracle_run(const void *input, void *target, int32_t *signal,
                    const int32_t *send_counts, int32_t *recv_counts, int32_t P, int32_t S,
                    int64_t in_slab, int64_t tgt_slab, int64_t core_num, int32_t dtype,
                    int64_t capacity);
int a2av_oracle_run_blocked(const void *input, void *target, int32_t *signal,
                            const int32_t *send_counts, int32_t *recv_counts, int32_t P,
                            int32_t S, int64_t in_slab, int64_t tgt_slab, int64_t core_num,
                            int32_t dtype, int64_t capacity, int32_t nblk);
int a2av_oracle_run_bias(const void *input, void *target, int32_t *signal,
                         const int32_t *send_counts, int32_t *recv_counts, int32_t P, int32_t S,
                         int64_t in_slab, int64_t tgt_slab, int64_t core_num, int32_t dtype,
                         int64_t capacity, int32_t nblk, const void *bias, int32_t hidden);
int a2av_oracle_run_indexed(const void *input, void *target, int32_t *signal,
                            const int32_t *send_counts, int32_t *recv_counts,
                            const int32_t *index, int32_t P, int32_t S, int64_t in_slab,
                            int64_t tgt_slab, int64_t core_num, int32_t dtype, int64_t capacity,
                            int32_t row_elems, int64_t index_stride);

#define HIP_OK(x)                                                                         \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)

/* Inputs only: SplitMix64. */
static uint64_t rng;
static uint64_t next_u64(void)
{
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

enum { PLAIN = 0, BLOCKED = 1, INDEXED = 2, BIAS = 3, HOSTC = 4, NOALLOC = 5 };

typedef struct {
    const char *name;
    int kind;
    int32_t P;
    int32_t dtype;
    int64_t core_num;
    int32_t max_units; /* a count is 0..max_units units */
    int32_t unit;      /* elements per unit: nblk (blocked), row_elems (indexed),
                          nblk * hidden (bias), else 1 */
    int64_t chunk;     /* chunk_limit_bytes, 0 = default */
    int32_t nblk;      /* bias: sub-blocks per segment */
    int32_t hidden;    /* bias: row length */
    int32_t host;      /* blocked, bias, indexed: 1 = the *_host_counts entry point */
} Case;

static const Case kCases[] = {
    {"plain_fp32_cooperative", PLAIN, 8, A2AV_FP32, 64, 3000, 1, 0, 0, 0, 0},
    {"plain_int8_one_block", PLAIN, 4, A2AV_INT8, 1, 9000, 1, 0, 0, 0, 0},
    {"plain_int8_chunked", PLAIN, 5, A2AV_INT8, 10, 40000, 1, 65536, 0, 0, 0},
    {"plain_fp32_p64", PLAIN, 64, A2AV_FP32, 256, 300, 1, 0, 0, 0, 0},
    {"blocked_fp32_nblk4", BLOCKED, 8, A2AV_FP32, 16, 300, 4, 0, 0, 0, 0},
    {"indexed_int8_rows448", INDEXED, 8, A2AV_INT8, 64, 12, 448, 0, 0, 0, 0},
    {"bias_bf16_nblk2_h64", BIAS, 8, A2AV_BF16, 16, 10, 2 * 64, 0, 2, 64, 0},
    {"bias_fp16_nblk3_h24_chunked", BIAS, 5, A2AV_FP16, 5, 12, 3 * 24, 1024, 3, 24, 0},
    {"host_counts_fp32_chunked", HOSTC, 6, A2AV_FP32, 12, 5000, 1, 16384, 0, 0, 0},
    {"noalloc_int8_cooperative", NOALLOC, 8, A2AV_INT8, 64, 9000, 1, 0, 0, 0, 0},
    {"blocked_int8_nblk3_host_counts_chunked", BLOCKED, 6, A2AV_INT8, 12, 2000, 3, 4096, 0, 0, 1},
    {"bias_bf16_nblk2_h16_host_counts_chunked", BIAS, 4, A2AV_BF16, 8, 10, 2 * 16, 1024, 2, 16,
     1},
    {"indexed_fp32_rows5_host_counts_chunked", INDEXED, 5, A2AV_FP32, 10, 20, 5, 4096, 0, 0, 1},
};

/* A finite 16-bit value: random sign and mantissa, exponent kept well inside
 * the type's range (no NaN, infinity or overflow in the sums). */
static uint16_t finite16(int32_t dtype)
{
    const uint64_t r = next_u64();
    const uint16_t sign = (uint16_t)((r >> 20) & 1u) << 15;
    if (dtype == A2AV_BF16)
        return (uint16_t)(sign | (uint16_t)((100 + r % 55) << 7) | (uint16_t)((r >> 8) & 0x7Fu));
    return (uint16_t)(sign | (uint16_t)((5 + r % 20) << 10) | (uint16_t)((r >> 8) & 0x3FFu));
}

static int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

static int run_case(const Case *c, uint64_t seed)
{
    const int32_t P = c->P;
    const int64_t e = c->dtype == A2AV_FP32 ? 4 : c->dtype == A2AV_INT8 ? 1 : 2;
    rng = seed;

    int32_t *counts = malloc(sizeof(int32_t) * (size_t)(P * P));
    int64_t max_row = 0, max_col = 0;
    for (int32_t i = 0; i < P * P; ++i) {
        int32_t n = (int32_t)(next_u64() % (uint64_t)(c->max_units + 1));
        if (next_u64() % 5 == 0) n = 0;
        counts[i] = n * c->unit;
    }
    for (int32_t s = 0; s < P; ++s) {
        int64_t row = 0, col = 0;
        for (int32_t d = 0; d < P; ++d) {
            row += counts[s * P + d];
            col += counts[d * P + s];
        }
        if (row > max_row) max_row = row;
        if (col > max_col) max_col = col;
    }
    int64_t table_rows = 0, stride = 0;
    int64_t in_slab = round16(max_row * e) + 32;
    if (c->kind == INDEXED) {
        stride = max_row / c->unit + 2;
        table_rows = max_row / c->unit + 3;
        in_slab = table_rows * c->unit * e;
    }
    const int64_t tgt_slab = round16(max_col * e) + 48; /* a tail the run must not touch */
    const int64_t B = a2av_blocks(P, c->core_num);
    const int32_t S = (int32_t)B + 1;

    const size_t in_bytes = (size_t)(P * in_slab), tgt_bytes = (size_t)(P * tgt_slab);
    const size_t sig_bytes = sizeof(int32_t) * (size_t)P * (size_t)S;
    const size_t cnt_bytes = sizeof(int32_t) * (size_t)(P * P);
    const size_t idx_bytes = sizeof(int32_t) * (size_t)(P * (stride > 0 ? stride : 1));
    const size_t nbias = c->kind == BIAS ? (size_t)P * (size_t)c->nblk * (size_t)c->hidden : 1;
    const size_t bias_bytes = nbias * (c->dtype == A2AV_BF16 ? 4u : 2u);
    uint8_t *h_in = malloc(in_bytes), *h_tgt = malloc(tgt_bytes), *o_tgt = malloc(tgt_bytes);
    int32_t *h_sig = calloc((size_t)P * (size_t)S, sizeof(int32_t));
    int32_t *o_sig = calloc((size_t)P * (size_t)S, sizeof(int32_t));
    int32_t *h_recv = malloc(cnt_bytes), *o_recv = malloc(cnt_bytes);
    int32_t *h_idx = malloc(idx_bytes);
    if (c->kind == BIAS) {
        for (size_t i = 0; i + 1 < in_bytes; i += 2) {
            const uint16_t v = finite16(c->dtype);
            memcpy(h_in + i, &v, 2);
        }
    } else {
        for (size_t i = 0; i < in_bytes; ++i) h_in[i] = (uint8_t)next_u64();
    }
    uint8_t *h_bias = malloc(bias_bytes);
    for (size_t i = 0; i < nbias && c->kind == BIAS; ++i) {
        if (c->dtype == A2AV_BF16) {
            const float b = (float)((int64_t)(next_u64() % 64000u) - 32000) / 1000.0f;
            memcpy(h_bias + 4 * i, &b, 4);
        } else {
            const uint16_t b = finite16(A2AV_FP16);
            memcpy(h_bias + 2 * i, &b, 2);
        }
    }
    memset(o_tgt, 0xA5, tgt_bytes);
    for (int32_t i = 0; i < P * P; ++i) o_recv[i] = -7;
    for (int64_t i = 0; i < P * (stride > 0 ? stride : 1); ++i)
        h_idx[i] = table_rows > 0 ? (int32_t)(next_u64() % (uint64_t)table_rows) : 0;

    void *d_in, *d_tgt, *d_sig, *d_send, *d_recv, *d_idx, *d_bias, *d_status;
    HIP_OK(hipMalloc(&d_in, in_bytes));
    HIP_OK(hipMalloc(&d_tgt, tgt_bytes));
    HIP_OK(hipMalloc(&d_sig, sig_bytes));
    HIP_OK(hipMalloc(&d_send, cnt_bytes));
    HIP_OK(hipMalloc(&d_recv, cnt_bytes));
    HIP_OK(hipMalloc(&d_idx, idx_bytes));
    HIP_OK(hipMalloc(&d_bias, bias_bytes));
    HIP_OK(hipMalloc(&d_status, sizeof(int32_t)));
    HIP_OK(hipMemcpy(d_in, h_in, in_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_tgt, o_tgt, tgt_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sig, o_sig, sig_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_send, counts, cnt_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_recv, o_recv, cnt_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_idx, h_idx, idx_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_bias, h_bias, bias_bytes, hipMemcpyHostToDevice));

    a2av_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.device = 0;
    cfg.P = P;
    cfg.in_slab_bytes = in_slab;
    cfg.tgt_slab_bytes = tgt_slab;
    cfg.S = S;
    cfg.chunk_limit_bytes = c->chunk;
    a2av_handle *h = NULL;
    int st = a2av_create(&h, &cfg);
    if (st != A2AV_OK) {
        fprintf(stderr, "%s: a2av_create: %s\n", c->name, a2av_status_string(st));
        exit(2);
    }
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int gpu_st = A2AV_OK;
    for (int run = 0; run < 2 && gpu_st == A2AV_OK; ++run) {
        if (c->kind == PLAIN)
            gpu_st = a2av_run(h, d_in, d_tgt, d_sig, d_send, d_recv, P, c->core_num, c->dtype,
                              stream);
        else if (c->kind == HOSTC)
            gpu_st = a2av_run_host_counts(h, d_in, d_tgt, d_sig, d_send, d_recv, counts, P,
                                          c->core_num, c->dtype, stream);
        else if (c->kind == NOALLOC)
            gpu_st = a2av_run_noalloc(d_in, d_tgt, d_sig, d_send, d_recv, (int32_t *)d_status, P,
                                      in_slab, tgt_slab, S, c->core_num, c->dtype, stream);
        else if (c->kind == BLOCKED && c->host)
            gpu_st = a2av_run_blocked_host_counts(h, d_in, d_tgt, d_sig, d_send, d_recv, counts,
                                                  P, c->core_num, c->dtype, c->unit, stream);
        else if (c->kind == BLOCKED)
            gpu_st = a2av_run_blocked(h, d_in, d_tgt, d_sig, d_send, d_recv, P, c->core_num,
                                      c->dtype, c->unit, stream);
        else if (c->kind == BIAS && c->host)
            gpu_st = a2av_run_bias_host_counts(h, d_in, d_tgt, d_sig, d_send, d_recv, d_bias,
                                               counts, P, c->core_num, c->dtype, c->nblk,
                                               c->hidden, stream);
        else if (c->kind == BIAS)
            gpu_st = a2av_run_bias(h, d_in, d_tgt, d_sig, d_send, d_recv, d_bias, P, c->core_num,
                                   c->dtype, c->nblk, c->hidden, stream);
        else if (c->host)
            gpu_st = a2av_run_indexed_host_counts(h, d_in, d_tgt, d_sig, d_send, d_recv, d_idx,
                                                  counts, P, c->core_num, c->dtype, c->unit,
                                                  stride, stream);
        else
            gpu_st = a2av_run_indexed(h, d_in, d_tgt, d_sig, d_send, d_recv, d_idx, P,
                                      c->core_num, c->dtype, c->unit, stride, stream);
        if (gpu_st != A2AV_OK)
            fprintf(stderr, "%s: run %d: %s (%s)\n", c->name, run, a2av_status_string(gpu_st),
                    a2av_last_hip_error(h));
        HIP_OK(hipStreamSynchronize(stream));
        if (gpu_st == A2AV_OK && c->kind == NOALLOC) {
            int32_t dev_st = -1;
            HIP_OK(hipMemcpy(&dev_st, d_status, sizeof(dev_st), hipMemcpyDeviceToHost));
            gpu_st = dev_st;
        } else if (gpu_st == A2AV_OK) {
            gpu_st = a2av_query_error(h);
        }
    }
    HIP_OK(hipMemcpy(h_tgt, d_tgt, tgt_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_sig, d_sig, sig_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_recv, d_recv, cnt_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(stream));
    a2av_destroy(h);

    int o_st = 0;
    for (int run = 0; run < 2 && o_st == 0; ++run) {
        if (c->kind == PLAIN || c->kind == HOSTC || c->kind == NOALLOC)
            o_st = a2av_oracle_run(h_in, o_tgt, o_sig, counts, o_recv, P, S, in_slab, tgt_slab,
                                   c->core_num, c->dtype, 0);
        else if (c->kind == BLOCKED)
            o_st = a2av_oracle_run_blocked(h_in, o_tgt, o_sig, counts, o_recv, P, S, in_slab,
                                           tgt_slab, c->core_num, c->dtype, 0, c->unit);
        else if (c->kind == BIAS)
            o_st = a2av_oracle_run_bias(h_in, o_tgt, o_sig, counts, o_recv, P, S, in_slab,
                                        tgt_slab, c->core_num, c->dtype, 0, c->nblk, h_bias,
                                        c->hidden);
        else
            o_st = a2av_oracle_run_indexed(h_in, o_tgt, o_sig, counts, o_recv, h_idx, P, S,
                                           in_slab, tgt_slab, c->core_num, c->dtype, 0, c->unit,
                                           stride);
    }

    int ok = 1;
    if (gpu_st != A2AV_OK) {  /* every case is a valid exchange */
        fprintf(stderr, "%s: status %d (%s), expected A2AV_OK\n", c->name, gpu_st,
                a2av_status_string(gpu_st));
        ok = 0;
    }
    if (gpu_st != o_st) {
        fprintf(stderr, "%s: status %d, oracle %d\n", c->name, gpu_st, o_st);
        ok = 0;
    }
    if (memcmp(h_tgt, o_tgt, tgt_bytes) != 0) {
        size_t i = 0;
        while (h_tgt[i] == o_tgt[i]) ++i;
        fprintf(stderr, "%s: target differs, first at byte %zu\n", c->name, i);
        ok = 0;
    }
    if (memcmp(h_sig, o_sig, sig_bytes) != 0) {
        fprintf(stderr, "%s: signal differs\n", c->name);
        ok = 0;
    }
    if (memcmp(h_recv, o_recv, cnt_bytes) != 0) {
        fprintf(stderr, "%s: recv_counts differ\n", c->name);
        ok = 0;
    }
    printf("%s: P=%d B=%lld payload-bound %lld bytes: %s\n", c->name, (int)P, (long long)B,
           (long long)(max_row * e), ok ? "ok" : "MISMATCH");
    fflush(stdout);

    HIP_OK(hipFree(d_in));
    HIP_OK(hipFree(d_tgt));
    HIP_OK(hipFree(d_sig));
    HIP_OK(hipFree(d_send));
    HIP_OK(hipFree(d_recv));
    HIP_OK(hipFree(d_idx));
    HIP_OK(hipFree(d_bias));
    HIP_OK(hipFree(d_status));
    free(counts);
    free(h_in);
    free(h_tgt);
    free(o_tgt);
    free(h_sig);
    free(o_sig);
    free(h_recv);
    free(o_recv);
    free(h_idx);
    free(h_bias);
    return ok;
}

int main(void)
{
    int all = 1;
    for (size_t k = 0; k < sizeof(kCases) / sizeof(kCases[0]); ++k)
        all &= run_case(&kCases[k], 1000 + k);
    printf("%s\n", all ? "all cases match the oracle" : "MISMATCH");
    return all ? 0 : 1;
}
