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
// One wave per (token, row segment).  Lanes j < k fetch slot and weight of
// expert j once and broadcast them as scalars.  A lane owns VPL 16-byte
// vectors of the segment and issues all K * VPL loads before any arithmetic
// (VPL shrinks as K grows to keep ~32 loads in flight per lane); it then
// accumulates in fp32 with one fused multiply-add per expert in top-k order
// (acc starts at +0) and rounds to bf16 (RNE).  The fixed order makes the
// result identical on every run.  Expert rows and the output are streamed
// with non-temporal loads/stores.  Slots outside [0, E*C) are skipped, which
// is also how dropped (over-capacity) pairs are handled.
#include <hip/hip_ext.h>

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

// Loads in flight per lane ~ K * VPL <= 32.
constexpr int vpl_for(int K) { return K <= 4 ? 8 : (K <= 8 ? 4 : 2); }

template <int K, int VPL>
hipError_t launch_vpl(const uint16_t *y, int64_t nrows, int nvec, const int32_t *token_slot, const float *w,
                      int64_t T, uint16_t *out, hipStream_t s, hipEvent_t start, hipEvent_t stop)
{
    const int segs = (nvec + VPL * kWave - 1) / (VPL * kWave);
    const int64_t blocks = (T * segs + kWavesPerBlock - 1) / kWavesPerBlock;
    if (!grid_fits(blocks, kBlock))
        return hipErrorInvalidConfiguration;
    if (start || stop)
        hipExtLaunchKernelGGL((combine_kernel<K, VPL>), dim3((unsigned)blocks), dim3(kBlock), 0, s, start, stop, 0,
                              (const u32x4 *)y, nrows, nvec, token_slot, w, T, segs, (u32x4 *)out);
    else
        hipLaunchKernelGGL((combine_kernel<K, VPL>), dim3((unsigned)blocks), dim3(kBlock), 0, s, (const u32x4 *)y,
                           nrows, nvec, token_slot, w, T, segs, (u32x4 *)out);
    return hipGetLastError();
}

template <int K>
hipError_t launch(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w, int64_t T,
                  uint16_t *out, hipStream_t s, hipEvent_t start, hipEvent_t stop)
{
    constexpr int V = vpl_for(K);
    const int nvec = H / 8;
    // few tokens: one vector per lane so that enough waves are in flight
    const int64_t waves_wide = T * ((nvec + V * kWave - 1) / (V * kWave));
    if (waves_wide < 2048)
        return launch_vpl<K, 1>(y, nrows, nvec, token_slot, w, T, out, s, start, stop);
    return launch_vpl<K, V>(y, nrows, nvec, token_slot, w, T, out, s, start, stop);
}

}  // namespace

bool combine_grid_fits(int64_t T, int H, int k)
{
    if (k < 1 || k > 16)
        return false;
    const int nvec = H / 8, V = vpl_for(k);
    const int64_t segs_wide = (nvec + V * kWave - 1) / (V * kWave);
    const int64_t segs = T * segs_wide < 2048 ? (nvec + kWave - 1) / kWave : segs_wide;
    return grid_fits((T * segs + kWavesPerBlock - 1) / kWavesPerBlock, kBlock);
}

hipError_t launch_combine(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                          int64_t T, int k, uint16_t *out, hipStream_t s, hipEvent_t start, hipEvent_t stop)
{
    switch (k) {
#define MOE_COMBINE_K(K) \
    case K: return launch<K>(y, nrows, H, token_slot, w, T, out, s, start, stop);
    MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
    MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
    MOE_COMBINE_K(9) MOE_COMBINE_K(10) MOE_COMBINE_K(11) MOE_COMBINE_K(12)
    MOE_COMBINE_K(13) MOE_COMBINE_K(14) MOE_COMBINE_K(15) MOE_COMBINE_K(16)
#undef MOE_COMBINE_K
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
