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
// the maximum, and the lowest lane holding that maximum wins.  Because lanes
// hold consecutive experts and each lane offers its lowest index among
// equals, "lowest winning lane" is "lowest expert", which is the tie rule.
// Logits are compared through an order-preserving 32-bit key (sign-magnitude
// to unsigned), with -0 mapped to +0 so the two compare equal.
//
// The group reductions stay in the VALU: DPP quad permutes and row mirrors
// reduce within each 16-lane row; a whole-wave group (G = 64) then combines
// the four row results as scalars (readlane), so the winner's lane, its
// index and the maximum are wave-uniform SGPR values.  The softmax
// denominator is summed in a fixed order, so results do not depend on
// scheduling.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over aligned groups of G <= 16 lanes, result in every lane of the group.
template <int G>
__device__ __forceinline__ uint32_t row_max(uint32_t v)
{
    if (G >= 2) v = umax(v, dpp<kDppQuadXor1>(v));
    if (G >= 4) v = umax(v, dpp<kDppQuadXor2>(v));
    if (G >= 8) v = umax(v, dpp<kDppHalfMirror>(v));
    if (G >= 16) v = umax(v, dpp<kDppMirror>(v));
    return v;
}

template <int G>
__device__ __forceinline__ float row_sum(float v)
{
    if (G >= 2) v += dpp<kDppQuadXor1>(v);
    if (G >= 4) v += dpp<kDppQuadXor2>(v);
    if (G >= 8) v += dpp<kDppHalfMirror>(v);
    if (G >= 16) v += dpp<kDppMirror>(v);
    return v;
}

// Group max for any G: rows by DPP, then across rows.
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
    v = row_max<(G < 16 ? G : 16)>(v);
    if (G == 32)
        v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
    if (G == 64) {
        const uint32_t a = umax((uint32_t)lane_value((int)v, 0), (uint32_t)lane_value((int)v, 16));
        const uint32_t b = umax((uint32_t)lane_value((int)v, 32), (uint32_t)lane_value((int)v, 48));
        v = umax(a, b);
    }
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    v = row_sum<(G < 16 ? G : 16)>(v);
    if (G == 32)
        v += __shfl_xor(v, 16);
    if (G == 64)
        v = (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
    return v;
}

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

// VEC: the row's VPL consecutive logits of a lane are one aligned vector
// load (E % VPL == 0 and a suitably aligned base).
template <int G, int VPL, bool VEC>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float *__restrict__ logits, int64_t T, int E, int k,
                                                            int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w)
{
    static_assert(G >= 1 && G <= kWave && (kWave % G) == 0, "group must divide the wave");
    static_assert(VPL == 1 || G == kWave, "several logits per lane only with one token per wave");
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = wave * kGroupsPerWave + grp;
    const bool active = t < T;

    float v[VPL];
    uint32_t key[VPL];
    const float *row = logits + (active ? t : 0) * (int64_t)E + gl * VPL;
    if (VEC && active && gl * VPL < E) {
        if (VPL == 2) {
            const float2 p = *(const float2 *)row;
            v[0] = p.x;
            v[VPL > 1 ? 1 : 0] = p.y;
        } else {
#pragma unroll
            for (int i = 0; i < VPL; i += 4) {
                const float4 p = *(const float4 *)(row + i);
                v[i] = p.x;
                v[(i + 1) % VPL] = p.y;
                v[(i + 2) % VPL] = p.z;
                v[(i + 3) % VPL] = p.w;
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            key[i] = order_key(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const bool ok = active && gl * VPL + i < E;
            v[i] = ok ? row[i] : 0.0f;
            key[i] = ok ? order_key(v[i]) : 0u;  // 0 is below every real key
        }
    }

    float top = 0.0f;   // the largest logit of the token
    int my_e = 0;       // lane gl == j keeps the j-th choice
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
        int wl, e;
        if (G == kWave) {
            wl = __ffsll((unsigned long long)ball) - 1;    // wave-uniform
            e = wl * VPL + lane_value(bi, wl);
        } else {
            const uint64_t gmask = (ball >> (grp * G)) & ((1ull << (G % kWave)) - 1ull);
            wl = __ffsll((unsigned long long)gmask) - 1;   // per group
            e = wl;                                          // VPL == 1
        }
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
            my_e = e;
            my_v = val;
        }
    }

    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (active && gl * VPL + i < E)
            s += expf(v[i] - top);
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
    const bool vec = VPL > 1 && E % VPL == 0 && (VPL == 2 ? ((uintptr_t)logits % 8 == 0)
                                                           : (E % 4 == 0 && (uintptr_t)logits % 16 == 0));
    if (vec)
        hipLaunchKernelGGL((route_topk_kernel<G, VPL, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, logits, T,
                           E, k, idx, w);
    else
        hipLaunchKernelGGL((route_topk_kernel<G, VPL, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, logits, T,
                           E, k, idx, w);
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
