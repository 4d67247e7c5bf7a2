// route_topk.hip -- router top-k selection and softmax weights (gfx950).
//
// pplx blog "Efficient and portable mixture-of-experts communication",
// Introduction: the router yields a probability distribution over experts,
// the experts with the top-K scores are chosen and weighted by it.
// "How GPUs Talk to Each Other During LLM Inference", section 7: each
// expert's output is weighted by the router's score for that expert.
//
// One token per group of G lanes (G a power of two dividing 64); lane l of a
// group holds the VPL consecutive logits l*VPL .. l*VPL+VPL-1.  Selection
// runs k rounds: every lane offers its best remaining logit, the group takes
// the maximum with a butterfly, and the lowest lane holding that maximum
// wins.  Because lanes hold consecutive experts and each lane offers its
// lowest index among equals, "lowest winning lane" is "lowest expert", which
// is the tie rule.  Logits are compared through an order-preserving 32-bit
// key (sign-magnitude to unsigned), with -0 mapped to +0 so the two compare
// equal.  The softmax denominator is a fixed-order sum, so results do not
// depend on scheduling.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0)
        u = 0;  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key)
{
    return (key & 0x80000000u) ? __uint_as_float(key & 0x7FFFFFFFu) : __uint_as_float(~key);
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
        uint32_t other = (uint32_t)__shfl_xor((int)v, o);
        v = other > v ? other : v;
    }
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <int G, int VPL>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float *__restrict__ logits, int64_t T,
                                                            int E, int k, int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w)
{
    static_assert(G >= 1 && G <= kWave && (kWave % G) == 0, "group must divide the wave");
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = wave * kGroupsPerWave + grp;
    const bool active = t < T;

    float v[VPL];
    uint32_t key[VPL];
    const float *row = logits + (active ? t : 0) * (int64_t)E;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = gl * VPL + i;
        const bool ok = active && e < E;
        v[i] = ok ? row[e] : 0.0f;
        key[i] = ok ? order_key(v[i]) : 0u;  // 0 is below every real key
    }

    float top = 0.0f;     // the largest logit of the token
    int my_e = 0;         // lane gl == j keeps the j-th choice
    float my_v = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            if (key[i] > bk) {  // strict: the lowest index among equals
                bk = key[i];
                bi = i;
            }
        }
        const uint32_t gm = group_max<G>(bk);
        const uint64_t ball = __ballot(bk == gm);
        const uint64_t gmask = (G == kWave) ? ball : ((ball >> (grp * G)) & ((1ull << (G % kWave)) - 1ull));
        const int wl = __ffsll((unsigned long long)gmask) - 1;   // lowest lane holding the max
        const int wbi = __shfl(bi, grp * G + wl);
        if (gl == wl) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (i == bi)
                    key[i] = 0u;
        }
        const float val = key_value(gm);
        if (j == 0)
            top = val;
        if (gl == j) {
            my_e = wl * VPL + wbi;
            my_v = val;
        }
    }

    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = gl * VPL + i;
        if (active && e < E)
            s += expf(v[i] - top);
    }
    s = group_sum<G>(s);

    if (active && gl < k) {
        topk_idx[t * k + gl] = my_e;
        topk_w[t * k + gl] = expf(my_v - top) / s;
    }
}

template <int G, int VPL>
hipError_t launch(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w, hipStream_t s)
{
    constexpr int64_t tokens_per_block = (int64_t)kWavesPerBlock * (kWave / G);
    const int64_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL((route_topk_kernel<G, VPL>), dim3((unsigned)blocks), dim3(kBlock), 0, s, logits, T, E,
                       k, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                             hipStream_t s)
{
    if (E <= 1) return launch<1, 1>(logits, T, E, k, idx, w, s);
    if (E <= 2) return launch<2, 1>(logits, T, E, k, idx, w, s);
    if (E <= 4) return launch<4, 1>(logits, T, E, k, idx, w, s);
    if (E <= 8) return launch<8, 1>(logits, T, E, k, idx, w, s);
    if (E <= 16) return launch<16, 1>(logits, T, E, k, idx, w, s);
    if (E <= 32) return launch<32, 1>(logits, T, E, k, idx, w, s);
    if (E <= 64) return launch<64, 1>(logits, T, E, k, idx, w, s);
    if (E <= 128) return launch<64, 2>(logits, T, E, k, idx, w, s);
    if (E <= 256) return launch<64, 4>(logits, T, E, k, idx, w, s);
    if (E <= 512) return launch<64, 8>(logits, T, E, k, idx, w, s);
    return launch<64, 16>(logits, T, E, k, idx, w, s);
}

}  // namespace moe
