/*
 * c_abi_example.c -- libmoe_route.so used from plain C99, with no Python and
 * no torch: one route + dispatch call, then combine with identity experts
 * (each slot's expert output is its dispatched row), on a seeded batch; then
 * the group-limited router, the separate dispatch call with E4M3 rows, and
 * the packed dispatch, on a second batch.  Every result is checked against
 * the CPU oracle's library.
 *
 * Test infrastructure: built by build(), run by tests/test_gpu_c_abi.py.
 * Prints "c-abi ok" and exits 0 when everything matches; otherwise prints
 * what differs and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_route.h"

/* the oracle's entry points (oracle/moe_oracle.c) */
int oracle_route_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *idx, float *w);
int oracle_assign_slots(const int32_t *idx, int64_t T, int32_t E, int32_t k, int32_t C, int32_t *counts,
                        int32_t *token_slot, int32_t *recv_src);
int oracle_combine(const uint16_t *y_pairs, const int32_t *token_slot, const float *w, int64_t T, int32_t k,
                   int32_t H, uint16_t *out, float *acc_out);
int oracle_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t k, int32_t G, int32_t M,
                              int32_t *idx, float *w);
int oracle_assign_packed(const int32_t *idx, int64_t T, int32_t E, int32_t k, int32_t *offsets,
                         int32_t *token_slot, int32_t *recv_src);
int oracle_quantize_rows_fp8(const uint16_t *x, int64_t n, int32_t H, uint8_t *codes, float *scales);

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static uint32_t next_u32(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s;
}

/* Second batch: 64 experts in 8 groups (3 kept), top-4, H = 256.  Route with
 * moe_route_topk_grouped; dispatch those ids with moe_dispatch as E4M3 rows
 * into fixed slots, and with moe_dispatch_packed as bf16 rows.  Returns the
 * number of values that differ from the oracle, or -1 on a failed call. */
static int grouped_fp8_packed(void)
{
    const int64_t T = 300;
    const int32_t E = 64, k = 4, H = 256, C = 300, G = 8, M = 3;
    const size_t nx = (size_t)T * H, np = (size_t)T * k, nrows = (size_t)E * C, nblk = H / 128;
    uint32_t seed = 777u;
    float *logits = malloc(sizeof(float) * T * E);
    uint16_t *x = malloc(2 * nx);
    for (int64_t i = 0; i < T * E; ++i)
        logits[i] = (float)((int)(next_u32(&seed) >> 8) % 4001 - 2000) / 500.0f;
    for (size_t i = 0; i < nx; ++i) {
        const uint32_t r = next_u32(&seed);
        x[i] = (uint16_t)(((r >> 31) << 15) | ((118u + (r >> 8) % 14u) << 7) | (r & 0x7Fu));
    }
    float *d_logits, *d_w, *d_scales;
    uint16_t *d_x, *d_prows;
    uint8_t *d_codes;
    int32_t *d_idx, *d_src, *d_counts, *d_slot, *d_psrc, *d_offs, *d_pslot;
    void *d_ws;
    const size_t ws = moe_dispatch_workspace_bytes(T, E, k);
    CHECK_HIP(hipMalloc((void **)&d_logits, sizeof(float) * T * E));
    CHECK_HIP(hipMalloc((void **)&d_x, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_idx, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_w, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_codes, nrows * H));
    CHECK_HIP(hipMalloc((void **)&d_scales, 4 * nrows * nblk));
    CHECK_HIP(hipMalloc((void **)&d_src, 4 * nrows));
    CHECK_HIP(hipMalloc((void **)&d_counts, 4 * E));
    CHECK_HIP(hipMalloc((void **)&d_slot, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_prows, 2 * np * H));
    CHECK_HIP(hipMalloc((void **)&d_psrc, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_offs, 4 * (E + 1)));
    CHECK_HIP(hipMalloc((void **)&d_pslot, 4 * np));
    CHECK_HIP(hipMalloc(&d_ws, ws));
    CHECK_HIP(hipMemcpy(d_logits, logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, 2 * nx, hipMemcpyHostToDevice));

    int rc = moe_route_topk_grouped(d_logits, T, E, k, G, M, d_idx, d_w, NULL);
    if (rc == MOE_OK)
        rc = moe_dispatch(d_x, T, H, d_idx, E, k, C, MOE_DTYPE_FP8_E4M3, d_codes, d_scales, d_src, d_counts, d_slot,
                          d_ws, ws, NULL);
    if (rc == MOE_OK)
        rc = moe_dispatch_packed(d_x, T, H, d_idx, E, k, MOE_DTYPE_BF16, d_prows, NULL, d_psrc, d_offs, d_pslot,
                                 d_ws, ws, NULL);
    if (rc != MOE_OK) {
        printf("second batch: %s\n", moe_status_string(rc));
        return -1;
    }
    CHECK_HIP(hipDeviceSynchronize());

    int32_t *idx = malloc(4 * np), *counts = malloc(4 * E), *slot = malloc(4 * np), *src = malloc(4 * nrows);
    int32_t *offs = malloc(4 * (E + 1)), *pslot = malloc(4 * np), *psrc = malloc(4 * np);
    float *w = malloc(4 * np), *scales = malloc(4 * nrows * nblk);
    uint8_t *codes = malloc(nrows * H);
    uint16_t *prows = malloc(2 * np * H);
    CHECK_HIP(hipMemcpy(idx, d_idx, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w, d_w, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_counts, 4 * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot, d_slot, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(src, d_src, 4 * nrows, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(codes, d_codes, nrows * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(scales, d_scales, 4 * nrows * nblk, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(offs, d_offs, 4 * (E + 1), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(pslot, d_pslot, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(psrc, d_psrc, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(prows, d_prows, 2 * np * H, hipMemcpyDeviceToHost));

    int32_t *o_idx = malloc(4 * np), *o_counts = malloc(4 * E), *o_slot = malloc(4 * np), *o_src = malloc(4 * nrows);
    int32_t *o_offs = malloc(4 * (E + 1)), *o_pslot = malloc(4 * np), *o_psrc = malloc(4 * np);
    float *o_w = malloc(4 * np), *o_scales = malloc(4 * nx / 128);
    uint8_t *o_codes = malloc(nx);
    if (oracle_route_topk_grouped(logits, T, E, k, G, M, o_idx, o_w) ||
        oracle_assign_slots(o_idx, T, E, k, C, o_counts, o_slot, o_src) ||
        oracle_assign_packed(o_idx, T, E, k, o_offs, o_pslot, o_psrc) ||
        oracle_quantize_rows_fp8(x, T, H, o_codes, o_scales)) {
        printf("oracle refused the second batch\n");
        return -1;
    }
    int bad = 0;
    for (size_t i = 0; i < np; ++i) {
        bad += idx[i] != o_idx[i] || slot[i] != o_slot[i] || pslot[i] != o_pslot[i] || psrc[i] != o_psrc[i];
        bad += fabs((double)w[i] - o_w[i]) > ldexp(fabs(o_w[i]), -17);
    }
    for (int e = 0; e < E; ++e)
        bad += counts[e] != o_counts[e];
    for (int e = 0; e <= E; ++e)
        bad += offs[e] != o_offs[e];
    /* every filled slot: its source token, that token's E4M3 codes and block
     * scales (fixed slots), and its bf16 row (packed rows) */
    for (size_t p = 0; p < np; ++p) {
        const int64_t t = (int64_t)(p / k);
        const int32_t s = o_slot[p], r = o_pslot[p];
        if (s >= 0) {
            bad += src[s] != t;
            bad += memcmp(codes + (size_t)s * H, o_codes + (size_t)t * H, H) != 0;
            bad += memcmp(scales + (size_t)s * nblk, o_scales + (size_t)t * nblk, 4 * nblk) != 0;
        }
        bad += memcmp(prows + (size_t)r * H, x + (size_t)t * H, 2 * (size_t)H) != 0;
    }
    hipFree(d_logits); hipFree(d_x); hipFree(d_idx); hipFree(d_w); hipFree(d_codes); hipFree(d_scales);
    hipFree(d_src); hipFree(d_counts); hipFree(d_slot); hipFree(d_prows); hipFree(d_psrc); hipFree(d_offs);
    hipFree(d_pslot); hipFree(d_ws);
    free(logits); free(x); free(idx); free(counts); free(slot); free(src); free(offs); free(pslot); free(psrc);
    free(w); free(scales); free(codes); free(prows); free(o_idx); free(o_counts); free(o_slot); free(o_src);
    free(o_offs); free(o_pslot); free(o_psrc); free(o_w); free(o_scales); free(o_codes);
    if (bad)
        printf("second batch: %d values differ from the oracle\n", bad);
    return bad;
}

int main(void)
{
    const int64_t T = 300;
    const int32_t E = 8, k = 2, H = 256, C = 300;
    const size_t nx = (size_t)T * H, np = (size_t)T * k, nrows = (size_t)E * C;
    uint32_t seed = 12345u;

    float *logits = malloc(sizeof(float) * T * E);
    uint16_t *x = malloc(2 * nx);
    for (int64_t i = 0; i < T * E; ++i)
        logits[i] = (float)((int)(next_u32(&seed) >> 8) % 2001 - 1000) / 250.0f;
    for (size_t i = 0; i < nx; ++i) {     /* finite bf16 values of magnitude 2^-7 .. 2^3 */
        const uint32_t r = next_u32(&seed);
        x[i] = (uint16_t)(((r >> 31) << 15) | ((120u + (r >> 8) % 10u) << 7) | (r & 0x7Fu));
    }

    float *d_logits, *d_w;
    uint16_t *d_x, *d_recv, *d_out;
    int32_t *d_idx, *d_src, *d_counts, *d_slot;
    void *d_ws;
    const size_t ws = moe_dispatch_workspace_bytes(T, E, k);
    CHECK_HIP(hipMalloc((void **)&d_logits, sizeof(float) * T * E));
    CHECK_HIP(hipMalloc((void **)&d_x, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_idx, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_w, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_recv, 2 * nrows * H));
    CHECK_HIP(hipMalloc((void **)&d_src, 4 * nrows));
    CHECK_HIP(hipMalloc((void **)&d_counts, 4 * E));
    CHECK_HIP(hipMalloc((void **)&d_slot, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_out, 2 * nx));
    CHECK_HIP(hipMalloc(&d_ws, ws));
    CHECK_HIP(hipMemcpy(d_logits, logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, 2 * nx, hipMemcpyHostToDevice));

    int rc = moe_route_dispatch(d_logits, T, E, k, d_x, H, C, MOE_DTYPE_BF16, d_idx, d_w, d_recv, NULL, d_src,
                                d_counts, d_slot, d_ws, ws, NULL);
    if (rc != MOE_OK) {
        printf("moe_route_dispatch: %s\n", moe_status_string(rc));
        return 1;
    }
    /* identity experts: the dispatched rows are the expert outputs */
    rc = moe_combine(d_recv, E, C, H, d_slot, d_w, T, k, d_out, NULL);
    if (rc != MOE_OK) {
        printf("moe_combine: %s\n", moe_status_string(rc));
        return 1;
    }
    if (moe_combine(d_recv, E, C, H, d_slot, d_w, T, 17, d_out, NULL) != MOE_ERR_UNSUPPORTED) {
        printf("k = 17 was not refused\n");
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());

    int32_t *idx = malloc(4 * np), *counts = malloc(4 * E), *slot = malloc(4 * np);
    float *w = malloc(4 * np);
    uint16_t *out = malloc(2 * nx);
    CHECK_HIP(hipMemcpy(idx, d_idx, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w, d_w, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_counts, 4 * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot, d_slot, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out, 2 * nx, hipMemcpyDeviceToHost));

    int32_t *o_idx = malloc(4 * np), *o_counts = malloc(4 * E), *o_slot = malloc(4 * np),
            *o_src = malloc(4 * nrows);
    float *o_w = malloc(4 * np);
    uint16_t *y_pairs = calloc(np * H, 2), *o_out = malloc(2 * nx);
    if (oracle_route_topk(logits, T, E, k, o_idx, o_w) || oracle_assign_slots(o_idx, T, E, k, C, o_counts, o_slot,
                                                                              o_src)) {
        printf("oracle refused the inputs\n");
        return 1;
    }
    int bad = 0;
    for (size_t i = 0; i < np; ++i) {
        bad += idx[i] != o_idx[i] || slot[i] != o_slot[i];
        bad += fabs((double)w[i] - o_w[i]) > ldexp(fabs(o_w[i]), -17);
    }
    for (int e = 0; e < E; ++e)
        bad += counts[e] != o_counts[e];
    /* combine of the oracle: pair (t, j) reads row x[t] when it has a slot */
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
            if (o_slot[t * k + j] >= 0)
                memcpy(y_pairs + (size_t)(t * k + j) * H, x + (size_t)t * H, 2 * (size_t)H);
    oracle_combine(y_pairs, o_slot, w, T, k, H, o_out, NULL);
    for (size_t i = 0; i < nx; ++i)
        bad += out[i] != o_out[i];
    if (bad) {
        printf("%d values differ from the oracle\n", bad);
        return 1;
    }
    hipFree(d_logits); hipFree(d_x); hipFree(d_idx); hipFree(d_w); hipFree(d_recv);
    hipFree(d_src); hipFree(d_counts); hipFree(d_slot); hipFree(d_out); hipFree(d_ws);
    if (grouped_fp8_packed() != 0)
        return 1;
    printf("c-abi ok\n");
    return 0;
}
