/*
 * moe_oracle.c -- plain, slow CPU oracle for MoE token routing, dispatch and
 * combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library; both sides implement the definitions below independently.
 *
 * Sources (web pages; cited by title and section):
 *   [PPLX]  Perplexity, "Efficient and portable mixture-of-experts
 *           communication" (pplx-kernels blog, 2025): sections Introduction,
 *           Portable kernels, Dispatch, Combine.
 *   [GPUS]  "How GPUs Talk to Each Other During LLM Inference", section 7
 *           (Expert Parallelism).
 *   [HBK]   AI-infra handbook, "NVSHMEM and DeepEP: GPU-initiated
 *           communication": sections "Why MoE's all-to-all is hard",
 *           "High-throughput mode" (FP8 dispatch / BF16 combine bullet),
 *           "Low-latency mode" (fixed slots).
 *
 * Precision: selection compares the fp32 logits exactly; softmax weights are
 * computed in fp64 and rounded once to fp32; fp8 quantisation is decided in
 * fp32 (the precision the codes are defined in); combine accumulates in fp32
 * with one fused multiply-add per expert in top-k order, then rounds to bf16.
 *
 * Built with: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -lm
 * Every function is single-threaded.  Return 0 on success, -1 on a bad
 * argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32: widening is exact. */
static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even.  For a finite value the
 * 16 dropped bits are rounded by adding 0x7FFF plus the lowest kept bit (a
 * tie then carries only when the kept part is odd).  Overflow carries into
 * the exponent and yields infinity, as IEEE rounding does.  NaN stays a
 * (quiet) NaN with its sign. */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, so the largest
 * finite magnitude is 1.75 * 2^8 = 448.  Exponent field 0 encodes the
 * subnormals m * 2^-9.
 *
 * Encoding rounds to nearest with ties to even and saturates: any finite
 * magnitude above 448 becomes 448.  The rounding is done on the exact
 * scaled significand with rint() in the default round-to-nearest-even mode;
 * all scalings are by powers of two and therefore exact. */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a > 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: count in units of 2^-9; 8 units is the smallest
         * normal 2^-6, whose code is also 8. */
        double units = rint(ldexp(a, 9));
        return (uint8_t)(sign | (uint8_t)units);
    }
    int ex;
    frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;         /* a = 1.xxx * 2^e, e in [-6, 8] */
    double m = rint(ldexp(a, 3 - e));   /* significand in eighths, [8, 16] */
    if (m == 16.0) {
        m = 8.0;
        e += 1;
    }
    int code = ((e + 7) << 3) | ((int)m - 8);
    if (code > 0x7E)        /* would be the NaN pattern: saturate */
        code = 0x7E;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* Route: top-k experts and their router weights                             */
/* [PPLX] Introduction: the router yields a probability distribution, the    */
/* experts with the top-K scores are chosen, and the output is the sum of    */
/* expert outputs times weights taken from that distribution.  [GPUS] 7: the */
/* router picks 8 of 256 experts; each output is weighted by the router's    */
/* score for that expert.                                                    */
/* ------------------------------------------------------------------------ */

/* For each token t (row of logits[T][E]):
 *   idx[t][j], j = 0..k-1: the k experts with the largest logits, in
 *     descending logit order; equal logits are ordered by ascending expert
 *     index (IEEE comparison, so -0 and +0 are equal).
 *   w[t][j] = softmax over all E logits, evaluated at expert idx[t][j]:
 *     exp(L[e] - max) / sum_e' exp(L[e'] - max), in double, summed in
 *     ascending expert order, rounded once to float.  No renormalisation
 *     over the chosen k. */
int oracle_route_topk(const float *logits, int64_t T, int32_t E, int32_t k,
                      int32_t *idx, float *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    if (T == 0)
        return 0;
    if (!logits || !idx || !w)
        return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!taken)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * (int64_t)E;
        memset(taken, 0, (size_t)E);
        /* repeated selection of the largest remaining logit */
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || row[e] > row[best])   /* strict: lower index wins ties */
                    best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = best;
        }
        double mx = (double)row[0];
        for (int32_t e = 1; e < E; ++e)
            if ((double)row[e] > mx)
                mx = (double)row[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e)
            z += exp((double)row[e] - mx);
        for (int32_t j = 0; j < k; ++j)
            w[t * k + j] = (float)(exp((double)row[idx[t * k + j]] - mx) / z);
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Route, group-limited ("node-limited") variant                             */
/* [HBK] "High-throughput mode": DeepSeek-V3 limits each token to a few      */
/* nodes -- every node is scored by the sum of its two best expert scores,   */
/* only the best nodes stay eligible, and the top experts are then picked    */
/* among those nodes' experts.  Here a node is a group of E/G consecutive    */
/* experts and a score is the expert's logit (the value experts are          */
/* selected on).                                                             */
/* ------------------------------------------------------------------------ */

/* For each token t:
 *   score[g], g = 0..G-1: the fp32 sum of the two largest logits among
 *     experts g*E/G .. (g+1)*E/G - 1 (a repeated largest value counts twice).
 *   kept groups: the M groups with the largest scores, equal scores ordered
 *     by ascending group index.
 *   idx[t][j]: the k largest logits among the kept groups' experts, ordered
 *     as in oracle_route_topk (descending, ties to the lower index).
 *   w[t][j]: the full softmax over all E logits at idx[t][j], exactly as in
 *     oracle_route_topk: limiting the groups changes which experts are
 *     chosen, not the router's distribution.
 * Requires E % G == 0, E/G >= 2, 1 <= M <= G, k <= M*E/G. */
int oracle_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t k, int32_t G, int32_t M,
                              int32_t *idx, float *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E || G < 1 || E % G != 0 || E / G < 2 || M < 1 || M > G ||
        (int64_t)k > (int64_t)M * (E / G))
        return -1;
    if (T == 0)
        return 0;
    if (!logits || !idx || !w)
        return -1;
    const int32_t gs = E / G;
    float *score = (float *)malloc((size_t)G * sizeof(float));
    unsigned char *kept = (unsigned char *)malloc((size_t)G);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!score || !kept || !taken) {
        free(score);
        free(kept);
        free(taken);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * (int64_t)E;
        /* group scores: largest, then largest of the rest */
        for (int32_t g = 0; g < G; ++g) {
            const int32_t lo = g * gs;
            int32_t b1 = lo;
            for (int32_t e = lo + 1; e < lo + gs; ++e)
                if (row[e] > row[b1])
                    b1 = e;
            int32_t b2 = -1;
            for (int32_t e = lo; e < lo + gs; ++e)
                if (e != b1 && (b2 < 0 || row[e] > row[b2]))
                    b2 = e;
            const float a = row[b1], b = row[b2];
            score[g] = a + b;                       /* one fp32 rounding */
        }
        /* the M best groups, repeated selection (strict: lower index wins) */
        memset(kept, 0, (size_t)G);
        for (int32_t m = 0; m < M; ++m) {
            int32_t best = -1;
            for (int32_t g = 0; g < G; ++g)
                if (!kept[g] && (best < 0 || score[g] > score[best]))
                    best = g;
            kept[best] = 1;
        }
        /* top-k among the kept groups' experts */
        for (int32_t e = 0; e < E; ++e)
            taken[e] = kept[e / gs] ? 0 : 1;      /* a banned expert is never eligible */
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || row[e] > row[best])
                    best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = best;
        }
        double mx = (double)row[0];
        for (int32_t e = 1; e < E; ++e)
            if ((double)row[e] > mx)
                mx = (double)row[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e)
            z += exp((double)row[e] - mx);
        for (int32_t j = 0; j < k; ++j)
            w[t * k + j] = (float)(exp((double)row[idx[t * k + j]] - mx) / z);
    }
    free(score);
    free(kept);
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch, step 1+2: per-expert counts and fixed-slot assignment           */
/* [HBK] "Why MoE's all-to-all is hard": route, then sort by destination,    */
/* then count per destination.  [HBK] "Low-latency mode": a fixed number of  */
/* slots per expert lets the sender compute its write address without a     */
/* count exchange.  [PPLX] Dispatch: the receiver packs tokens into          */
/* contiguous per-expert buffers for the grouped GEMM and keeps each token's */
/* source index for combine.  Within an expert, slots are filled in          */
/* ascending source-token order (the pages leave the order open).            */
/* ------------------------------------------------------------------------ */

/* Inputs: idx[T][k] (each row k distinct experts in [0, E)), capacity C.
 * Outputs:
 *   counts[e]           true number of (t, j) with idx[t][j] == e
 *                       (may exceed C: that is the overflow signal)
 *   token_slot[t][j]    e*C + r, r = number of earlier tokens routed to e,
 *                       or -1 when r >= C (dropped)
 *   recv_src[e*C + r]   t for every filled slot; -1 for unfilled slots
 * Walks tokens in ascending order and j ascending, handing out the next free
 * slot of each expert. */
int oracle_assign_slots(const int32_t *idx, int64_t T, int32_t E, int32_t k,
                        int32_t C, int32_t *counts, int32_t *token_slot,
                        int32_t *recv_src)
{
    if (T < 0 || E < 1 || k < 1 || k > E || C < 1)
        return -1;
    if (!counts || !recv_src || (T > 0 && (!idx || !token_slot)))
        return -1;
    int64_t *fill = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!fill)
        return -1;
    for (int64_t s = 0; s < (int64_t)E * C; ++s)
        recv_src[s] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E) {
                free(fill);
                return -1;
            }
            int64_t r = fill[e]++;
            if (r < C) {
                int64_t s = (int64_t)e * C + r;
                recv_src[s] = (int32_t)t;
                token_slot[t * k + j] = (int32_t)s;
            } else {
                token_slot[t * k + j] = -1;
            }
        }
    }
    for (int32_t e = 0; e < E; ++e)
        counts[e] = (int32_t)fill[e];
    free(fill);
    return 0;
}

/* Packed, count-sized layout.  [HBK] "High-throughput mode": the number of
 * tokens bound for each destination is computed first and the receive
 * buffer is sized by it.  [PPLX] Dispatch: each expert's tokens are
 * contiguous for the grouped GEMM.  Here every expert's rows follow the
 * previous expert's, with no reserved slack:
 *   offsets[e]   pairs routed to experts 0 .. e-1 (exclusive prefix of the
 *                per-expert counts); offsets[E] = T*k
 *   token_slot[t][j] = offsets[e] + r, where (t, j) is the r-th pair routed
 *                to e = idx[t][j] in ascending token order
 *   recv_src[row] = t for every row 0 .. T*k-1
 * Inputs: idx[T][k] (each row k distinct experts in [0, E)). */
int oracle_assign_packed(const int32_t *idx, int64_t T, int32_t E, int32_t k, int32_t *offsets,
                         int32_t *token_slot, int32_t *recv_src)
{
    if (T < 0 || E < 1 || k < 1 || k > E || !offsets || (T > 0 && (!idx || !token_slot || !recv_src)))
        return -1;
    int64_t *count = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *fill = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!count || !fill) {
        free(count);
        free(fill);
        return -1;
    }
    for (int64_t p = 0; p < T * k; ++p) {
        const int32_t e = idx[p];
        if (e < 0 || e >= E) {
            free(count);
            free(fill);
            return -1;
        }
        ++count[e];
    }
    int64_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        offsets[e] = (int32_t)run;
        run += count[e];
    }
    offsets[E] = (int32_t)run;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            const int32_t e = idx[t * k + j];
            const int64_t row = offsets[e] + fill[e]++;
            token_slot[t * k + j] = (int32_t)row;
            recv_src[row] = (int32_t)t;
        }
    }
    free(count);
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch, step 3: packing rows                                            */
/* [HBK] "High-throughput mode": FP8 for dispatch with one scale per 128     */
/* elements, BF16 for combine.  [HBK] simulation listing: the FP8 row is the */
/* hidden vector plus one fp32 scale per 128 elements.                       */
/* ------------------------------------------------------------------------ */

/* Quantise one bf16 row of H elements (H a multiple of 128) to E4M3 codes
 * with one fp32 scale per block of 128:
 *   amax = max |x_i| over the block (exact, in float)
 *   sc   = amax / 448 (IEEE float division), or 1 when amax == 0
 *   q_i  = E4M3 encode of (x_i / sc) (IEEE float division), RNE, saturating */
int oracle_quantize_row_fp8(const uint16_t *x, int32_t H, uint8_t *codes,
                            float *scales)
{
    if (H < 128 || H % 128 != 0 || !x || !codes || !scales)
        return -1;
    for (int32_t b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int32_t i = 0; i < 128; ++i) {
            float a = fabsf(bf16_bits_to_float(x[b * 128 + i]));
            if (a > amax)
                amax = a;
        }
        float sc = (amax == 0.0f) ? 1.0f : amax / 448.0f;
        scales[b] = sc;
        for (int32_t i = 0; i < 128; ++i) {
            float q = bf16_bits_to_float(x[b * 128 + i]) / sc;
            codes[b * 128 + i] = oracle_e4m3_encode(q);
        }
    }
    return 0;
}

/* Number of filled slots: sum over experts of min(counts[e], C). */
int64_t oracle_filled_rows(const int32_t *counts, int32_t E, int32_t C)
{
    int64_t n = 0;
    for (int32_t e = 0; e < E; ++e)
        n += counts[e] < C ? counts[e] : C;
    return n;
}

/* Content of every filled slot, in ascending slot order (expert-major, then
 * rank), as a dense array of R = oracle_filled_rows() rows.  Row p is the
 * slot slot_of_row[p].
 *   dtype 0 (bf16): rows[p] = x[recv_src[slot]] bit for bit, 2H bytes
 *   dtype 1 (fp8):  rows[p] = E4M3 codes of x[recv_src[slot]] (H bytes) and
 *                   scales[p] = its H/128 block scales */
int oracle_pack(const uint16_t *x, int64_t T, int32_t H, int32_t dtype,
                const int32_t *recv_src, const int32_t *counts, int32_t E,
                int32_t C, void *rows, float *scales, int32_t *slot_of_row)
{
    if (T < 0 || H < 1 || E < 1 || C < 1 || (dtype != 0 && dtype != 1))
        return -1;
    if (dtype == 1 && (H % 128 != 0 || !scales))
        return -1;
    if (!recv_src || !counts || !slot_of_row)
        return -1;
    int64_t p = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t n = counts[e] < C ? counts[e] : C;
        for (int32_t r = 0; r < n; ++r, ++p) {
            int64_t s = (int64_t)e * C + r;
            int32_t t = recv_src[s];
            if (t < 0 || t >= T)
                return -1;
            slot_of_row[p] = (int32_t)s;
            const uint16_t *src = x + (int64_t)t * H;
            if (dtype == 0) {
                memcpy((uint16_t *)rows + p * H, src, (size_t)H * 2);
            } else {
                int rc = oracle_quantize_row_fp8(src, H, (uint8_t *)rows + p * H,
                                                 scales + p * (H / 128));
                if (rc)
                    return rc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* [PPLX] Combine: the receiver reads each expert's output, takes the weight */
/* from the routing table and forms the weighted sum into a caller-allocated */
/* tensor; outputs travel unquantised in 16 bits.  [GPUS] 7: the k weighted  */
/* outputs are added up at the token's origin.                               */
/* ------------------------------------------------------------------------ */

/* y_pairs[t*k + j][H]: the bf16 output of expert idx[t][j] for token t.
 * For each t and h:
 *   acc = +0.0f
 *   for j = 0..k-1 with token_slot[t][j] >= 0: acc = fmaf(w[t][j], y, acc)
 *   out[t][h] = bf16 round-to-nearest-even of acc
 * acc_out (optional, may be NULL) receives the float accumulators. */
int oracle_combine(const uint16_t *y_pairs, const int32_t *token_slot,
                   const float *w, int64_t T, int32_t k, int32_t H,
                   uint16_t *out, float *acc_out)
{
    if (T < 0 || k < 1 || H < 1)
        return -1;
    if (T == 0)
        return 0;
    if (!y_pairs || !token_slot || !w || !out)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                if (token_slot[t * k + j] < 0)
                    continue;
                float y = bf16_bits_to_float(y_pairs[(t * k + j) * (int64_t)H + h]);
                acc = fmaf(w[t * k + j], y, acc);
            }
            out[t * H + h] = oracle_bf16_round(acc);
            if (acc_out)
                acc_out[t * H + h] = acc;
        }
    }
    return 0;
}

/* bf16 nearest-even rounding of a double, in one step (no intermediate
 * float): 8 significant bits for normal magnitudes, a fixed step of 2^-133
 * below 2^-126; a magnitude that rounds above the largest finite bf16 is
 * infinite. */
static uint16_t bf16_round_double(double v)
{
    if (v != v)
        return 0x7FC0;
    const double a = fabs(v);
    double q;
    if (a < 0x1p-126) {
        q = rint(a * 0x1p133) * 0x1p-133;
    } else {
        int e;
        const double m = frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
        q = ldexp(rint(ldexp(m, 8)), e - 8);
    }
    uint16_t bits;
    if (q > 0x1.FEp127) {
        bits = 0x7F80;
    } else {
        const float f = (float)q;               /* exact: q has at most 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, 4);
        bits = (uint16_t)(u >> 16);
    }
    return (uint16_t)(bits | (signbit(v) ? 0x8000 : 0));
}

/* Array form of bf16_round_double (exposed so that its rounding can be
 * checked on its own). */
int oracle_bf16_round_double_n(const double *v, int64_t n, uint16_t *out)
{
    if (n < 0 || (n > 0 && (!v || !out)))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_round_double(v[i]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Combine epilogue: residual add and RMSNorm                                */
/* [GPUS] section 5: right after the sum, the result is added to the        */
/* residual stream (the updated residual is stored), and the updated stream  */
/* goes through the next module's RMSNorm -- x * rsqrt(mean of squares over  */
/* the token + eps) * gamma -- all before anything is written back.  Here    */
/* the sum is combine's weighted sum.                                        */
/* ------------------------------------------------------------------------ */

/* For each token t and h:
 *   acc = combine's fp32 accumulator (as oracle_combine: fmaf in top-k order)
 *   r[h] = acc + residual[t][h]             (one fp32 addition)
 *   residual_out[t][h] = bf16 RNE of r[h]
 *   ms = (sum over h of r[h]^2) / H         (double)
 *   normed_out[t][h] = bf16 RNE of r[h] / sqrt(ms + eps) * gamma[h], evaluated
 *                      in double and rounded once.
 * residual, gamma: bf16.  With eps = 0 an all-zero row is 0/0 (NaN). */
int oracle_combine_residual_rmsnorm(const uint16_t *y_pairs, const int32_t *token_slot, const float *w, int64_t T,
                                    int32_t k, int32_t H, const uint16_t *residual, const uint16_t *gamma,
                                    float eps, uint16_t *residual_out, uint16_t *normed_out)
{
    if (T < 0 || k < 1 || H < 1 || !(eps >= 0.0f))
        return -1;
    if (T == 0)
        return 0;
    if (!y_pairs || !token_slot || !w || !residual || !gamma || !residual_out || !normed_out)
        return -1;
    float *r = (float *)malloc((size_t)H * sizeof(float));
    if (!r)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                if (token_slot[t * k + j] < 0)
                    continue;
                const float y = bf16_bits_to_float(y_pairs[(t * k + j) * (int64_t)H + h]);
                acc = fmaf(w[t * k + j], y, acc);
            }
            r[h] = acc + bf16_bits_to_float(residual[t * H + h]);
            residual_out[t * H + h] = oracle_bf16_round(r[h]);
            ss += (double)r[h] * (double)r[h];
        }
        const double inv = 1.0 / sqrt(ss / H + (double)eps);
        for (int32_t h = 0; h < H; ++h)
            normed_out[t * H + h] = bf16_round_double((double)r[h] * inv * (double)bf16_bits_to_float(gamma[h]));
    }
    free(r);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Buffer sizing                                                             */
/* [HBK] simulation listing: an FP8 token is H bytes plus one fp32 scale per */
/* 128 elements.  [HBK] "Low-latency mode": a slot also carries a small      */
/* header; the receive buffer reserves slots for the worst case.             */
/* ------------------------------------------------------------------------ */

/* Bytes of one dispatched row: 2H for bf16; H + 4*(H/128) for fp8. */
int64_t oracle_row_bytes(int32_t H, int32_t dtype)
{
    return dtype == 0 ? 2 * (int64_t)H : (int64_t)H + 4 * (int64_t)(H / 128);
}

/* Bytes of a fixed-slot receive buffer: experts * slots * (row + header). */
int64_t oracle_fixed_slot_bytes(int64_t experts, int64_t slots_per_expert,
                                int32_t H, int32_t dtype, int32_t header_bytes)
{
    return experts * slots_per_expert * (oracle_row_bytes(H, dtype) + header_bytes);
}

/* Element-wise array forms of the two encoders above, for sweeps. */
void oracle_bf16_round_n(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

void oracle_e4m3_encode_n(const float *in, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(in[i]);
}

/* Quantise n rows of H elements, one oracle_quantize_row_fp8() per row. */
int oracle_quantize_rows_fp8(const uint16_t *x, int64_t n, int32_t H, uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < n; ++r) {
        int rc = oracle_quantize_row_fp8(x + r * H, H, codes + r * H, scales + r * (H / 128));
        if (rc)
            return rc;
    }
    return 0;
}
