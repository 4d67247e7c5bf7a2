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
// One wave per (token, column segment).  Lanes j < k fetch slot and weight
// of expert j once; every round then issues the k * kBatch 16-byte loads of
// the lane's vectors before any arithmetic, and accumulates in fp32 with one
// fused multiply-add per expert in top-k order (acc starts at +0), rounding
// to bf16 (RNE) at the end.  The fixed order makes the result identical on
// every run.  Slots outside [0, E*C) are skipped, which is also how dropped
// (over-capacity) pairs are handled.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBatch = 2;

template <int K>
__global__ __launch_bounds__(kBlock) void combine_kernel(const uint4 *__restrict__ y, int64_t nrows, int nvec,
                                                         const int32_t *__restrict__ token_slot,
                                                         const float *__restrict__ topk_w, int64_t T, int vpl,
                                                         int segs, uint4 *__restrict__ out)
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

    uint4 *dst = out + t * nvec;
    const int v0 = seg * vpl * kWave + lane;
    for (int i0 = 0; i0 < vpl; i0 += kBatch) {
        uint4 buf[K][kBatch];
#pragma unroll
        for (int j = 0; j < K; ++j) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int v = v0 + (i0 + b) * kWave;
                if (slot[j] >= 0 && i0 + b < vpl && v < nvec)
                    buf[j][b] = y[(int64_t)slot[j] * nvec + v];
                else
                    buf[j][b] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int v = v0 + (i0 + b) * kWave;
            if (!(i0 + b < vpl && v < nvec))
                continue;
            float acc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[q] = 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if (slot[j] < 0)
                    continue;
                const uint32_t u[4] = {buf[j][b].x, buf[j][b].y, buf[j][b].z, buf[j][b].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = __builtin_fmaf(wt[j], bf16_lo(u[q]), acc[2 * q]);
                    acc[2 * q + 1] = __builtin_fmaf(wt[j], bf16_hi(u[q]), acc[2 * q + 1]);
                }
            }
            dst[v] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        }
    }
}

template <int K>
hipError_t launch(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w, int64_t T,
                  uint16_t *out, hipStream_t s)
{
    const int nvec = H / 8;
    const int max_segs = (nvec + kWave - 1) / kWave;
    int64_t want = (2048 + T - 1) / T;
    int segs = (int)(want > max_segs ? max_segs : want);
    const int vpl = (nvec + segs * kWave - 1) / (segs * kWave);
    segs = (nvec + vpl * kWave - 1) / (vpl * kWave);
    const int64_t blocks = (T * segs + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(combine_kernel<K>, dim3((unsigned)blocks), dim3(kBlock), 0, s, (const uint4 *)y, nrows,
                       nvec, token_slot, w, T, vpl, segs, (uint4 *)out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                          int64_t T, int k, uint16_t *out, hipStream_t s)
{
    switch (k) {
    case 1: return launch<1>(y, nrows, H, token_slot, w, T, out, s);
    case 2: return launch<2>(y, nrows, H, token_slot, w, T, out, s);
    case 3: return launch<3>(y, nrows, H, token_slot, w, T, out, s);
    case 4: return launch<4>(y, nrows, H, token_slot, w, T, out, s);
    case 5: return launch<5>(y, nrows, H, token_slot, w, T, out, s);
    case 6: return launch<6>(y, nrows, H, token_slot, w, T, out, s);
    case 7: return launch<7>(y, nrows, H, token_slot, w, T, out, s);
    case 8: return launch<8>(y, nrows, H, token_slot, w, T, out, s);
    case 9: return launch<9>(y, nrows, H, token_slot, w, T, out, s);
    case 10: return launch<10>(y, nrows, H, token_slot, w, T, out, s);
    case 11: return launch<11>(y, nrows, H, token_slot, w, T, out, s);
    case 12: return launch<12>(y, nrows, H, token_slot, w, T, out, s);
    case 13: return launch<13>(y, nrows, H, token_slot, w, T, out, s);
    case 14: return launch<14>(y, nrows, H, token_slot, w, T, out, s);
    case 15: return launch<15>(y, nrows, H, token_slot, w, T, out, s);
    case 16: return launch<16>(y, nrows, H, token_slot, w, T, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
