/*
 * c_abi_example.c -- libmoe_route.so used from plain C99, with no Python and
 * no torch: one route + dispatch call, then combine with identity experts
 * (each slot's expert output is its dispatched row), on a seeded batch; then
 * the group-limited router, the separate dispatch call with E4M3 rows, and
 * the packed dispatch, on a second batch; then the plain router, the one-call
 * packed and no-alloc dispatches and the fused residual + RMSNorm epilogue
 * (bf16 and E4M3 output) on a third.  Every entry point runs, and every
 * result is checked against the CPU oracle's library.
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
int oracle_combine_residual_rmsnorm(const uint16_t *y_pairs, const int32_t *token_slot, const float *w, int64_t T,
                                    int32_t k, int32_t H, const uint16_t *residual, const uint16_t *gamma,
                                    float eps, uint16_t *residual_out, uint16_t *normed_out);

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

static int bf16_ulps(uint16_t a, uint16_t b)
{
    const int ia = (a & 0x8000) ? -(int)(a & 0x7FFF) : (int)(a & 0x7FFF);
    const int ib = (b & 0x8000) ? -(int)(b & 0x7FFF) : (int)(b & 0x7FFF);
    return ia > ib ? ia - ib : ib - ia;
}

/* Third batch: 16 experts, top-2, H = 384.  moe_route_topk; the one-call
 * packed dispatch and the one-call no-alloc dispatch, whose ids must be
 * moe_route_topk's; then combine with the fused residual + RMSNorm epilogue
 * over the packed rows (identity experts), in bf16 and with E4M3 output.
 * Returns the number of values that differ from the oracle, or -1. */
static int plain_packed_noalloc_epilogue(void)
{
    const int64_t T = 200;
    const int32_t E = 16, k = 2, H = 384, C = 200;
    const size_t nx = (size_t)T * H, np = (size_t)T * k, nrows = (size_t)E * C;
    const float eps = 1e-6f;
    uint32_t seed = 4242u;
    float *logits = malloc(sizeof(float) * T * E);
    uint16_t *x = malloc(2 * nx), *res = malloc(2 * nx), *gamma = malloc(2 * (size_t)H);
    for (int64_t i = 0; i < T * E; ++i)
        logits[i] = (float)((int)(next_u32(&seed) >> 8) % 2001 - 1000) / 300.0f;
    for (size_t i = 0; i < nx; ++i) {
        uint32_t r = next_u32(&seed);
        x[i] = (uint16_t)(((r >> 31) << 15) | ((119u + (r >> 8) % 12u) << 7) | (r & 0x7Fu));
        r = next_u32(&seed);
        res[i] = (uint16_t)(((r >> 31) << 15) | ((119u + (r >> 8) % 12u) << 7) | (r & 0x7Fu));
    }
    for (int32_t i = 0; i < H; ++i)   /* positive weights 0.5 .. 2 */
        gamma[i] = (uint16_t)(((126u + next_u32(&seed) % 2u) << 7) | (next_u32(&seed) & 0x7Fu));

    float *d_logits, *d_w, *d_w2, *d_w3, *d_nsc;
    uint16_t *d_x, *d_res, *d_gamma, *d_prows, *d_frows, *d_rout, *d_nout, *d_nout8;
    uint8_t *d_nq;
    int32_t *d_idx, *d_idx2, *d_idx3, *d_psrc, *d_offs, *d_pslot, *d_fsrc, *d_counts, *d_fslot;
    void *d_ws;
    const size_t ws = moe_dispatch_workspace_bytes(T, E, k);
    CHECK_HIP(hipMalloc((void **)&d_logits, sizeof(float) * T * E));
    CHECK_HIP(hipMalloc((void **)&d_x, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_res, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_gamma, 2 * (size_t)H));
    CHECK_HIP(hipMalloc((void **)&d_idx, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_idx2, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_idx3, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_w, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_w2, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_w3, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_prows, 2 * np * H));
    CHECK_HIP(hipMalloc((void **)&d_psrc, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_offs, 4 * (E + 1)));
    CHECK_HIP(hipMalloc((void **)&d_pslot, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_frows, 2 * nrows * H));
    CHECK_HIP(hipMalloc((void **)&d_fsrc, 4 * nrows));
    CHECK_HIP(hipMalloc((void **)&d_counts, 4 * E));
    CHECK_HIP(hipMalloc((void **)&d_fslot, 4 * np));
    CHECK_HIP(hipMalloc((void **)&d_rout, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_nout, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_nout8, 2 * nx));
    CHECK_HIP(hipMalloc((void **)&d_nq, nx));
    CHECK_HIP(hipMalloc((void **)&d_nsc, 4 * nx / 128));
    CHECK_HIP(hipMalloc(&d_ws, ws));
    CHECK_HIP(hipMemcpy(d_logits, logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, 2 * nx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_res, res, 2 * nx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_gamma, gamma, 2 * (size_t)H, hipMemcpyHostToDevice));

    int rc = moe_route_topk(d_logits, T, E, k, d_idx, d_w, NULL);
    if (rc == MOE_OK)
        rc = moe_route_dispatch_packed(d_logits, T, E, k, d_x, H, MOE_DTYPE_BF16, d_idx2, d_w2, d_prows, NULL,
                                       d_psrc, d_offs, d_pslot, d_ws, ws, NULL);
    if (rc == MOE_OK)
        rc = moe_route_dispatch_noalloc(d_logits, T, E, k, d_x, H, C, MOE_DTYPE_BF16, d_idx3, d_w3, d_frows, NULL,
                                        d_fsrc, d_counts, d_fslot, NULL);
    /* combine over the packed rows: one "expert" of T*k rows */
    if (rc == MOE_OK)
        rc = moe_combine_residual_rmsnorm(d_prows, 1, (int32_t)np, H, d_pslot, d_w, T, k, d_res, d_gamma, eps,
                                          d_rout, d_nout, NULL);
    if (rc == MOE_OK)
        rc = moe_combine_residual_rmsnorm_fp8(d_prows, 1, (int32_t)np, H, d_pslot, d_w, T, k, d_res, d_gamma, eps,
                                              d_rout, d_nout8, d_nq, d_nsc, NULL);
    if (rc != MOE_OK) {
        printf("third batch: %s\n", moe_status_string(rc));
        return -1;
    }
    CHECK_HIP(hipDeviceSynchronize());

    int32_t *idx = malloc(4 * np), *idx2 = malloc(4 * np), *idx3 = malloc(4 * np), *offs = malloc(4 * (E + 1));
    int32_t *pslot = malloc(4 * np), *psrc = malloc(4 * np), *counts = malloc(4 * E), *fslot = malloc(4 * np);
    int32_t *fsrc = malloc(4 * nrows);
    float *w = malloc(4 * np), *w2 = malloc(4 * np), *w3 = malloc(4 * np), *nsc = malloc(4 * nx / 128);
    uint16_t *prows = malloc(2 * np * H), *frows = malloc(2 * nrows * H), *rout = malloc(2 * nx),
             *nout = malloc(2 * nx), *nout8 = malloc(2 * nx);
    uint8_t *nq = malloc(nx);
    CHECK_HIP(hipMemcpy(idx, d_idx, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(idx2, d_idx2, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(idx3, d_idx3, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w, d_w, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w2, d_w2, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w3, d_w3, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(offs, d_offs, 4 * (E + 1), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(pslot, d_pslot, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(psrc, d_psrc, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_counts, 4 * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fslot, d_fslot, 4 * np, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fsrc, d_fsrc, 4 * nrows, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(prows, d_prows, 2 * np * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(frows, d_frows, 2 * nrows * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(rout, d_rout, 2 * nx, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(nout, d_nout, 2 * nx, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(nout8, d_nout8, 2 * nx, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(nq, d_nq, nx, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(nsc, d_nsc, 4 * nx / 128, hipMemcpyDeviceToHost));

    int32_t *o_idx = malloc(4 * np), *o_offs = malloc(4 * (E + 1)), *o_pslot = malloc(4 * np),
            *o_psrc = malloc(4 * np), *o_counts = malloc(4 * E), *o_fslot = malloc(4 * np),
            *o_fsrc = malloc(4 * nrows);
    float *o_w = malloc(4 * np), *o_sc = malloc(4 * nx / 128), *g_sc = malloc(4 * nx / 128);
    uint16_t *y_pairs = malloc(2 * np * H), *o_rout = malloc(2 * nx), *o_nout = malloc(2 * nx);
    uint8_t *o_q = malloc(nx), *g_q = malloc(nx);
    if (oracle_route_topk(logits, T, E, k, o_idx, o_w) || oracle_assign_packed(o_idx, T, E, k, o_offs, o_pslot, o_psrc) ||
        oracle_assign_slots(o_idx, T, E, k, C, o_counts, o_fslot, o_fsrc)) {
        printf("oracle refused the third batch\n");
        return -1;
    }
    for (size_t p = 0; p < np; ++p)   /* identity experts: pair (t, j) outputs x[t] */
        memcpy(y_pairs + p * H, x + (p / k) * H, 2 * (size_t)H);
    /* the epilogue's oracle takes the weights the kernel was given */
    if (oracle_combine_residual_rmsnorm(y_pairs, o_pslot, w, T, k, H, res, gamma, eps, o_rout, o_nout) ||
        oracle_quantize_rows_fp8(o_nout, T, H, o_q, o_sc) || oracle_quantize_rows_fp8(nout, T, H, g_q, g_sc)) {
        printf("oracle refused the third batch's epilogue\n");
        return -1;
    }
    int bad = 0;
    for (size_t i = 0; i < np; ++i) {
        bad += idx[i] != o_idx[i] || idx2[i] != idx[i] || idx3[i] != idx[i];
        bad += fabs((double)w[i] - o_w[i]) > ldexp(fabs(o_w[i]), -17);
        bad += memcmp(&w2[i], &w[i], 4) != 0 || memcmp(&w3[i], &w[i], 4) != 0;
        bad += pslot[i] != o_pslot[i] || psrc[i] != o_psrc[i] || fslot[i] != o_fslot[i];
        bad += memcmp(prows + (size_t)pslot[i] * H, x + (i / k) * H, 2 * (size_t)H) != 0;
        if (o_fslot[i] >= 0) {
            bad += fsrc[o_fslot[i]] != (int32_t)(i / k);
            bad += memcmp(frows + (size_t)o_fslot[i] * H, x + (i / k) * H, 2 * (size_t)H) != 0;
        }
    }
    for (int e = 0; e < E; ++e)
        bad += counts[e] != o_counts[e];
    for (int e = 0; e <= E; ++e)
        bad += offs[e] != o_offs[e];
    for (size_t i = 0; i < nx; ++i) {
        bad += rout[i] != o_rout[i];
        bad += bf16_ulps(nout[i], o_nout[i]) > 1;
        bad += nout8[i] != nout[i];
    }
    /* E4M3 output: a block whose normalised values equal the oracle's bit for
     * bit must carry the oracle's codes and scale; every block must carry the
     * encoding of the kernel's own normalised values */
    for (size_t b = 0; b < nx / 128; ++b) {
        const int same = memcmp(nout + b * 128, o_nout + b * 128, 256) == 0;
        bad += memcmp(nq + b * 128, g_q + b * 128, 128) != 0 || memcmp(&nsc[b], &g_sc[b], 4) != 0;
        if (same)
            bad += memcmp(nq + b * 128, o_q + b * 128, 128) != 0 || memcmp(&nsc[b], &o_sc[b], 4) != 0;
    }
    hipFree(d_logits); hipFree(d_x); hipFree(d_res); hipFree(d_gamma); hipFree(d_idx); hipFree(d_idx2);
    hipFree(d_idx3); hipFree(d_w); hipFree(d_w2); hipFree(d_w3); hipFree(d_prows); hipFree(d_psrc); hipFree(d_offs);
    hipFree(d_pslot); hipFree(d_frows); hipFree(d_fsrc); hipFree(d_counts); hipFree(d_fslot); hipFree(d_rout);
    hipFree(d_nout); hipFree(d_nout8); hipFree(d_nq); hipFree(d_nsc); hipFree(d_ws);
    free(logits); free(x); free(res); free(gamma); free(idx); free(idx2); free(idx3); free(offs); free(pslot);
    free(psrc); free(counts); free(fslot); free(fsrc); free(w); free(w2); free(w3); free(nsc); free(prows);
    free(frows); free(rout); free(nout); free(nout8); free(nq); free(o_idx); free(o_offs); free(o_pslot);
    free(o_psrc); free(o_counts); free(o_fslot); free(o_fsrc); free(o_w); free(o_sc); free(g_sc); free(y_pairs);
    free(o_rout); free(o_nout); free(o_q); free(g_q);
    if (bad)
        printf("third batch: %d values differ from the oracle\n", bad);
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
    if (grouped_fp8_packed() != 0 || plain_packed_noalloc_epilogue() != 0)
        return 1;
    printf("c-abi ok\n");
    return 0;
}
