// combine.hip -- gather each token's k expert outputs and form their
// router-weighted sum in the original token order (gfx950).
//
// pplx blog "Efficient and portable mixture-of-experts communication",
// Combine: the routing table says which buffer to read and which weight to
// apply for each expert; outputs travel unquantised in 16 bits and the
// weighted sum is written to a caller-allocated tensor.  "How GPUs Talk to
// Each Other During LLM Inference", section 7: the k weighted outputs are
// added up at the token's origin.
//
// Two launch shapes share one arithmetic.  combine_kernel: one wave per
// (token, row segment); a lane owns VPL 16-byte vectors of the segment and
// issues all K * VPL loads before any arithmetic (VPL shrinks as K grows to
// keep ~32 loads in flight per lane).  combine_row_kernel: one work-group per
// token, one thread per 16-byte vector of the row (up to 1024), K loads per
// lane; it balances better across the chip when the segmented launch would
// leave lanes idle or give too few waves per CU.  In both, lanes j < k fetch
// slot and weight of expert j once and broadcast them as scalars, and a lane
// accumulates in fp32 with one fused multiply-add per expert in top-k order
// (acc starts at +0) and rounds to bf16 (RNE).  The fixed order makes the
// result identical on every run.  Expert rows and the output are streamed
// with non-temporal loads/stores.  Slots outside [0, E*C) are skipped, which
// is also how dropped (over-capacity) pairs are handled.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int K, int VPL>
__global__ __launch_bounds__(kBlock) void combine_kernel(const u32x4 *__restrict__ y, int64_t nrows, int nvec,
                                                         const int32_t *__restrict__ token_slot,
                                                         const float *__restrict__ topk_w, int64_t T, int segs,
                                                         u32x4 *__restrict__ out)
{
    const int lane = lane_id();
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;

    int my_slot = -1;
    float my_w = 0.0f;
    if (lane < K) {
        const int s = token_slot[t * K + lane];
        my_slot = (s >= 0 && (int64_t)s < nrows) ? s : -1;
        my_w = topk_w[t * K + lane];
    }
    int slot[K];
    float wt[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        slot[j] = lane_value(my_slot, j);
        wt[j] = lane_value(my_w, j);
    }

    const int v0 = seg * VPL * kWave + lane;
    u32x4 buf[K][VPL];
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave;
            if (slot[j] >= 0 && v < nvec)
                buf[j][i] = __builtin_nontemporal_load(y + (int64_t)slot[j] * nvec + v);
            else
                buf[j][i] = (u32x4){0, 0, 0, 0};
        }
    }
    u32x4 *dst = out + t * nvec;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v0 + i * kWave;
        if (v >= nvec)
            continue;
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[q] = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (slot[j] < 0)
                continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(wt[j], bf16_lo(buf[j][i][q]), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(wt[j], bf16_hi(buf[j][i][q]), acc[2 * q + 1]);
            }
        }
        const u32x4 r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7])};
        __builtin_nontemporal_store(r, dst + v);
    }
}

// One work-group of blockDim.x >= nvec threads per token.  Every lane loads
// all K rows unconditionally (a skipped pair reads row 0, which exists since
// nrows >= 1, and is then left out of the sum): a load behind a wave-uniform
// branch would make the compiler wait for it before issuing the next one.
template <int K>
__global__ __launch_bounds__(1024) void combine_row_kernel(const u32x4 *__restrict__ y, int64_t nrows, int nvec,
                                                           const int32_t *__restrict__ token_slot,
                                                           const float *__restrict__ topk_w,
                                                           u32x4 *__restrict__ out)
{
    const int lane = lane_id();
    const int v = threadIdx.x;
    const int64_t t = blockIdx.x;

    int my_slot = -1;
    float my_w = 0.0f;
    if (lane < K) {
        const int s = token_slot[t * K + lane];
        my_slot = (s >= 0 && (int64_t)s < nrows) ? s : -1;
        my_w = topk_w[t * K + lane];
    }
    int slot[K];
    float wt[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        slot[j] = lane_value(my_slot, j);
        wt[j] = lane_value(my_w, j);
    }
    if (v >= nvec)
        return;

    u32x4 buf[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
        buf[j] = __builtin_nontemporal_load(y + (int64_t)(slot[j] >= 0 ? slot[j] : 0) * nvec + v);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (slot[j] < 0)
            continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __builtin_fmaf(wt[j], bf16_lo(buf[j][q]), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(wt[j], bf16_hi(buf[j][q]), acc[2 * q + 1]);
        }
    }
    const u32x4 r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                     pack_bf16x2(acc[6], acc[7])};
    __builtin_nontemporal_store(r, out + t * nvec + v);
}

// Loads in flight per lane ~ K * VPL <= 32.
constexpr int vpl_for(int K) { return K <= 4 ? 8 : (K <= 8 ? 4 : 2); }

// Launch shape for T tokens of nvec vectors (measured on MI355X; the row
// launch was 2-15% faster on every prefill shape tried except the one where
// the wide segments tile the row exactly and the launch has many waves, where
// it was ~2.5% slower).
struct Shape {
    int vpl;   // combine_kernel's VPL, or 0 for combine_row_kernel
    int bs;    // work-group size
    int segs;  // combine_kernel: segments per token
};

Shape choose_shape(int64_t T, int nvec, int k)
{
    const int V = vpl_for(k);
    const int segs_wide = (nvec + V * kWave - 1) / (V * kWave);
    const int64_t waves_wide = T * segs_wide;
    if (waves_wide < 2048)   // few tokens: one vector per lane so that enough waves are in flight
        return {1, kBlock, (nvec + kWave - 1) / kWave};
    const int row_bs = (nvec + kWave - 1) / kWave * kWave;
    const bool wide_exact = nvec % (V * kWave) == 0 && waves_wide >= 16384;
    if (row_bs <= 1024 && !wide_exact && grid_fits(T, row_bs))
        return {0, row_bs, 1};
    return {V, kBlock, segs_wide};
}

template <int K, int VPL>
hipError_t launch_vpl(const uint16_t *y, int64_t nrows, int nvec, const int32_t *token_slot, const float *w,
                      int64_t T, uint16_t *out, hipStream_t s)
{
    const int segs = (nvec + VPL * kWave - 1) / (VPL * kWave);
    const int64_t blocks = (T * segs + kWavesPerBlock - 1) / kWavesPerBlock;
    if (!grid_fits(blocks, kBlock))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((combine_kernel<K, VPL>), dim3((unsigned)blocks), dim3(kBlock), 0, s, (const u32x4 *)y,
                       nrows, nvec, token_slot, w, T, segs, (u32x4 *)out);
    return hipGetLastError();
}

template <int K>
hipError_t launch_row(const uint16_t *y, int64_t nrows, int nvec, const int32_t *token_slot, const float *w,
                      int64_t T, int bs, uint16_t *out, hipStream_t s)
{
    if (bs < nvec || bs > 1024 || !grid_fits(T, bs))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((combine_row_kernel<K>), dim3((unsigned)T), dim3(bs), 0, s, (const u32x4 *)y, nrows, nvec,
                       token_slot, w, (u32x4 *)out);
    return hipGetLastError();
}

template <int K>
hipError_t launch(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w, int64_t T,
                  uint16_t *out, hipStream_t s)
{
    constexpr int V = vpl_for(K);
    const int nvec = H / 8;
    const Shape sh = choose_shape(T, nvec, K);
    if (sh.vpl == 0)
        return launch_row<K>(y, nrows, nvec, token_slot, w, T, sh.bs, out, s);
    if (sh.vpl == 1)
        return launch_vpl<K, 1>(y, nrows, nvec, token_slot, w, T, out, s);
    return launch_vpl<K, V>(y, nrows, nvec, token_slot, w, T, out, s);
}

}  // namespace

bool combine_grid_fits(int64_t T, int H, int k)
{
    if (k < 1 || k > 16)
        return false;
    const Shape sh = choose_shape(T, H / 8, k);
    if (sh.vpl == 0)
        return grid_fits(T, sh.bs);
    return grid_fits((T * sh.segs + kWavesPerBlock - 1) / kWavesPerBlock, kBlock);
}

hipError_t launch_combine(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                          int64_t T, int k, uint16_t *out, hipStream_t s)
{
    switch (k) {
#define MOE_COMBINE_K(K) \
    case K: return launch<K>(y, nrows, H, token_slot, w, T, out, s);
    MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
    MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
    MOE_COMBINE_K(9) MOE_COMBINE_K(10) MOE_COMBINE_K(11) MOE_COMBINE_K(12)
    MOE_COMBINE_K(13) MOE_COMBINE_K(14) MOE_COMBINE_K(15) MOE_COMBINE_K(16)
#undef MOE_COMBINE_K
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
