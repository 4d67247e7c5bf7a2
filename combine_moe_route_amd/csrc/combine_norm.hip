// combine_norm.hip -- combine with its epilogue fused: residual add and
// RMSNorm (gfx950).
//
// "How GPUs Talk to Each Other During LLM Inference", section 5: right after
// a sum, the result is added to the residual stream (the updated stream is
// stored) and normalised by the next module's RMSNorm, x * rsqrt(mean of
// squares over the token + eps) * gamma, before anything else is written;
// the threads of a token combine their partial sums of squares.  Here the
// sum is combine's router-weighted sum (pplx blog, Combine), so one kernel
// replaces combine + add + norm and the token's row makes one trip.
//
// One work-group per token: 256 threads (512 for rows of 4097 to 8192
// elements, so each lane requests its whole share in one pass), or 1024 when
// there are too few tokens to fill the chip with 4-wave groups.  Thread i
// owns the row's 16-byte vectors i, i + BS, ... (NV of them).  In passes of
// P vectors it requests the k expert rows (non-temporal) and the residual,
// forms combine's fp32 accumulator exactly as combine_kernel does (fma per
// expert in top-k order from +0, dropped pairs skipped), adds the residual
// in fp32, stores the updated residual (bf16, nearest even) and keeps the
// fp32 sums in registers.  The norm is evaluated in double: the squares are summed in
// double (no fp32 underflow or overflow for any row: r^2 of a float spans
// 2^-298 .. 2^256), the work-group adds its wave totals in a fixed
// order, inv = 1 / sqrt(sum / H + eps) (IEEE double division and square
// root), and every kept value is written as (r * inv) * gamma rounded from
// double to bf16 in one step.  The only difference from an exact evaluation
// is the order of the double sum of squares.
//
// With Q the normalised row is also re-quantised for an fp8 consumer: the
// same E4M3 block encoding as dispatch's fp8 rows (handbook "NVSHMEM and
// DeepEP", "High-throughput mode"), applied to the bf16 normalised values.
// The 16 consecutive lanes (one DPP row) holding a 128-element block share
// its maximum through four DPP steps; each lane stores its 8 codes (8 bytes) and the
// block's first lane its scale.  The bf16 normalised row is then optional.
#include "device_common.hpp"
#include "fp8_e4m3.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ double wave_sum(double v)
{
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// bf16 bit pattern nearest (ties to even) to a double, rounded once.
// Magnitudes from 2^-126 up: round the 52-bit significand at bit 45 on the
// integer bit pattern and rebias the exponent (a carry into the exponent is
// the correct next binade; exponents past bf16's largest give infinity).
// Below 2^-126: bf16 subnormals are multiples of 2^-133, so the rounded
// multiple is rint(|v| * 2^133) (exact scaling, one rounding).
__device__ __forceinline__ uint32_t bf16_from_double(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    // both forms are computed and one selected: no branch per element
    const uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1ull)) >> 45;   // 11-bit exp, 7-bit frac
    const int64_t e = (int64_t)(r >> 7) - 1023 + 127;
    uint32_t mag = e >= 255 ? 0x7F80u : (uint32_t)(((uint64_t)e << 7) | (r & 0x7Full));
    mag = a > 0x7FF0000000000000ull ? 0x7FC0u : mag;                              // NaN
    const uint32_t sub = (uint32_t)__builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
    return sign | (a >= 0x3810000000000000ull ? mag : sub);                       // |v| >= 2^-126
}

template <int KMAX, int NV, int P, int BS, bool Q>
__global__ __launch_bounds__(BS) void combine_rmsnorm_kernel(
    const u32x4 *__restrict__ y, int64_t nrows, int nvec, const int32_t *__restrict__ token_slot,
    const float *__restrict__ topk_w, int k, const u32x4 *residual, const u32x4 *__restrict__ gamma, float eps,
    int H, u32x4 *residual_out, u32x4 *__restrict__ normed_out, u32x2 *__restrict__ normed_q,
    float *__restrict__ normed_scales)
{
    static_assert(BS % 16 == 0, "a 128-element block spans 16 consecutive threads");
    static_assert(NV % P == 0, "passes must tile the vectors");
    constexpr int kWaves = BS / kWave;
    __shared__ double part[kWaves];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = lane_id();

    int my_slot = -1;
    float my_w = 0.0f;
    if (lane < k) {
        const int s = token_slot[t * k + lane];
        my_slot = (s >= 0 && (int64_t)s < nrows) ? s : -1;
        my_w = topk_w[t * k + lane];
    }
    int slot[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        slot[j] = j < k ? lane_value(my_slot, j) : -1;
        wt[j] = j < k ? lane_value(my_w, j) : 0.0f;
    }

    const u32x4 *res_row = residual + t * nvec;
    u32x4 *res_out_row = residual_out + t * nvec;
    float r[NV][8];
    double ss = 0.0;
#pragma unroll
    for (int n0 = 0; n0 < NV; n0 += P) {
        u32x4 buf[KMAX][P];
        u32x4 rb[P];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int v = tid + (n0 + p) * BS;
                buf[j][p] = (slot[j] >= 0 && v < nvec) ? __builtin_nontemporal_load(y + (int64_t)slot[j] * nvec + v)
                                                       : (u32x4){0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int v = tid + (n0 + p) * BS;
            rb[p] = v < nvec ? __builtin_nontemporal_load(res_row + v) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int v = tid + (n0 + p) * BS;
            float acc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[q] = 0.0f;
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (slot[j] < 0)
                    continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = __builtin_fmaf(wt[j], bf16_lo(buf[j][p][q]), acc[2 * q]);
                    acc[2 * q + 1] = __builtin_fmaf(wt[j], bf16_hi(buf[j][p][q]), acc[2 * q + 1]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r[n0 + p][2 * q] = acc[2 * q] + bf16_lo(rb[p][q]);
                r[n0 + p][2 * q + 1] = acc[2 * q + 1] + bf16_hi(rb[p][q]);
            }
            if (v < nvec) {
                const u32x4 o = {pack_bf16x2(r[n0 + p][0], r[n0 + p][1]), pack_bf16x2(r[n0 + p][2], r[n0 + p][3]),
                                 pack_bf16x2(r[n0 + p][4], r[n0 + p][5]), pack_bf16x2(r[n0 + p][6], r[n0 + p][7])};
                __builtin_nontemporal_store(o, res_out_row + v);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    ss = __builtin_fma((double)r[n0 + p][q], (double)r[n0 + p][q], ss);
            }
        }
    }

    ss = wave_sum(ss);
    if (lane == 0)
        part[tid / kWave] = ss;
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
        total += part[i];
    const double inv = 1.0 / __builtin_sqrt(total / (double)H + (double)eps);

    u32x4 *out_row = normed_out + t * nvec;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int v = tid + n * BS;
        if (v >= nvec)
            continue;
        const u32x4 g = gamma[v];
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] = bf16_from_double(((double)r[n][2 * q] * inv) * (double)bf16_lo(g[q]));
            o[2 * q + 1] = bf16_from_double(((double)r[n][2 * q + 1] * inv) * (double)bf16_hi(g[q]));
        }
        const u32x4 w = {o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)};
        if (!Q || normed_out)
            __builtin_nontemporal_store(w, out_row + v);
        if (Q) {   // v < nvec holds for all 16 lanes of a block (nvec % 16 == 0, BS % 16 == 0)
            float f[8];
            float amax = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                f[q] = __uint_as_float(o[q] << 16);
                amax = fmaxf(amax, fabsf(f[q]));
            }
            amax = group_max<16>(amax);
            const float sc = block_scale(amax);
            __builtin_nontemporal_store(quantize8(f, sc), normed_q + t * nvec + v);
            if ((lane & 15) == 0)
                __builtin_nontemporal_store(sc, normed_scales + t * (nvec / 16) + v / 16);
        }
    }
}

// Outputs of one launch (pointers already offset to its first token).
struct NormOut {
    uint16_t *residual_out, *normed;   // normed may be NULL when q is set
    uint8_t *q;                         // NULL: no fp8 output
    float *scales;
};

template <int KMAX, int NV, int BS>
hipError_t launch_nv(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w, int64_t T,
                     int k, const uint16_t *residual, const uint16_t *gamma, float eps, NormOut o, hipStream_t s)
{
    // about 16 row loads in flight per lane
    constexpr int P0 = 16 / KMAX > 0 ? 16 / KMAX : 1;
    constexpr int P = P0 < NV ? P0 : NV;
    if (!grid_fits(T, BS))
        return hipErrorInvalidConfiguration;
#define MOE_NORM_LAUNCH(Q)                                                                                       \
    hipLaunchKernelGGL((combine_rmsnorm_kernel<KMAX, NV, P, BS, Q>), dim3((unsigned)T), dim3(BS), 0, s,          \
                       (const u32x4 *)y, nrows, H / 8, token_slot, w, k, (const u32x4 *)residual,               \
                       (const u32x4 *)gamma, eps, H, (u32x4 *)o.residual_out, (u32x4 *)o.normed, (u32x2 *)o.q, \
                       o.scales)
    if (o.q)
        MOE_NORM_LAUNCH(true);
    else
        MOE_NORM_LAUNCH(false);
#undef MOE_NORM_LAUNCH
    return hipGetLastError();
}

template <int KMAX>
hipError_t launch_k(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w, int64_t T,
                    int k, const uint16_t *residual, const uint16_t *gamma, float eps, NormOut o, hipStream_t s)
{
    const int nvec = H / 8;
#define MOE_NORM_NV(NV, BS) launch_nv<KMAX, NV, BS>(y, nrows, H, token_slot, w, T, k, residual, gamma, eps, o, s)
    if (T < 512) {      // fewer than 2048 waves with 4-wave groups: 16-wave groups, one pass for H <= 8192
        if (nvec <= 1024)
            return MOE_NORM_NV(1, 1024);
        return MOE_NORM_NV(2, 1024);
    }
    if (nvec <= kBlock)
        return MOE_NORM_NV(1, kBlock);
    if (nvec <= 2 * kBlock)
        return MOE_NORM_NV(2, kBlock);
    if (nvec <= 4 * kBlock)     // H <= 8192: 8-wave groups with all loads in one pass beat 4 vectors per lane
        return MOE_NORM_NV(2, 2 * kBlock);
    return MOE_NORM_NV(8, kBlock);
#undef MOE_NORM_NV
}

hipError_t launch_tokens(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                         int64_t T, int k, const uint16_t *residual, const uint16_t *gamma, float eps, NormOut o,
                         hipStream_t s)
{
    if (k <= 2)
        return launch_k<2>(y, nrows, H, token_slot, w, T, k, residual, gamma, eps, o, s);
    if (k <= 4)
        return launch_k<4>(y, nrows, H, token_slot, w, T, k, residual, gamma, eps, o, s);
    if (k <= 8)
        return launch_k<8>(y, nrows, H, token_slot, w, T, k, residual, gamma, eps, o, s);
    return launch_k<16>(y, nrows, H, token_slot, w, T, k, residual, gamma, eps, o, s);
}

}  // namespace

hipError_t launch_combine_rmsnorm(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                                  int64_t T, int k, const uint16_t *residual, const uint16_t *gamma, float eps,
                                  uint16_t *residual_out, uint16_t *normed_out, uint8_t *normed_q,
                                  float *normed_scales, hipStream_t s)
{
    // One work-group per token and at most 2^32 - 1 work-items per launch:
    // longer batches go in launches of 2^22 tokens (groups of at most 512
    // threads there).
    constexpr int64_t kPiece = int64_t(1) << 22;
    for (int64_t t0 = 0; t0 < T; t0 += kPiece) {
        const int64_t n = T - t0 < kPiece ? T - t0 : kPiece;
        const int64_t r = t0 * H;
        const NormOut o = {residual_out + r, normed_out ? normed_out + r : nullptr, normed_q ? normed_q + r : nullptr,
                           normed_scales ? normed_scales + t0 * (H / 128) : nullptr};
        const hipError_t e = launch_tokens(y, nrows, H, token_slot + t0 * k, w + t0 * k, n, k, residual + r, gamma,
                                           eps, o, s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace moe
