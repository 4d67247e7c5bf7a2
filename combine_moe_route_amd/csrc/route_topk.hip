// route_topk.hip -- router top-k selection and softmax weights (gfx950).
//
// pplx blog "Efficient and portable mixture-of-experts communication",
// Introduction: the router yields a probability distribution over experts,
// the experts with the top-K scores are chosen and weighted by it.
// "How GPUs Talk to Each Other During LLM Inference", section 7: each
// expert's output is weighted by the router's score for that expert.
//
// One token per group of G lanes (G a power of two dividing 64); lane l of a
// group holds the VPL consecutive logits l*VPL .. l*VPL+VPL-1 (for large E,
// 16-lane groups with up to 16 logits per lane: four tokens per wave).  Selection
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
#include "route_core.hpp"

namespace moe {
namespace {

using namespace route_core;

template <int G, int VPL, bool VEC>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float *__restrict__ logits, int64_t T, int E, int k,
                                                            int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w)
{
    static_assert(G >= 1 && G <= kWave && (kWave % G) == 0, "group must divide the wave");
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = wave * kGroupsPerWave + lane / G;
    const bool active = t < T;
    float v[VPL];
    uint32_t key[VPL];
    load_logits<VPL, VEC>(logits, t, active, E, lane % G, v, key);
    select_and_store<G, VPL>(v, key, active, t, E, k, topk_idx, topk_w);
}

// Router top-k for E <= 8 with the dispatch count step folded in.  A
// work-group routes 32 tokens (four waves of eight 8-lane groups) and, since
// it then holds every choice of those tokens, also records which of them
// chose each expert: masks[e * nchunks + c] has bit b set when token
// 32c + b routed to e (LDS atomic OR, which commutes, so the words do not
// depend on scheduling).  Dispatch derives counts, prefixes and in-chunk
// ranks from these words by popcount.
constexpr int kMaskChunk = 32;   // tokens per mask word

__global__ __launch_bounds__(kBlock) void route_topk_mask_kernel(const float *__restrict__ logits, int64_t T, int E,
                                                                 int k, int32_t *__restrict__ topk_idx,
                                                                 float *__restrict__ topk_w,
                                                                 uint32_t *__restrict__ masks, int nchunks)
{
    constexpr int G = 8;
    static_assert(kWavesPerBlock * (kWave / G) == kMaskChunk, "one work-group per mask word");
    __shared__ uint32_t smask[G];
    if (threadIdx.x < G)
        smask[threadIdx.x] = 0u;
    __syncthreads();
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = wave * (kWave / G) + lane / G;
    const bool active = t < T;
    float v[1];
    uint32_t key[1];
    load_logits<1, false>(logits, t, active, E, lane % G, v, key);
    const int my_e = select_and_store<G, 1>(v, key, active, t, E, k, topk_idx, topk_w);
    if (active && lane % G < k)
        atomicOr(&smask[my_e], 1u << (int)(t - (int64_t)blockIdx.x * kMaskChunk));
    __syncthreads();
    if ((int)threadIdx.x < E)
        masks[(int64_t)threadIdx.x * nchunks + blockIdx.x] = smask[threadIdx.x];
}

// Router top-k for E > 8 with the dispatch count step folded in, as above:
// a work-group routes 16 tokens with the plain router's lane layout for this
// E and T (so the weights are the same bits) and writes, for every expert,
// the 16-bit half of the 32-token membership word that covers its tokens
// (bit b of word c: token 32c + b chose e).  Each half is written by exactly
// one work-group, and when the halves are odd in number the last
// work-group also clears the unused upper half of the final word, so the
// words need no clearing beforehand and no global atomics.
constexpr int kHalfTokens = 16;

template <int G, int VPL, bool VEC>
__global__ __launch_bounds__(kHalfTokens * kWave) void route_topk_half_mask_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, uint16_t *__restrict__ half_masks, int nwords)
{
    extern __shared__ uint32_t hmask[];   // [E]
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hmask[e] = 0u;
    __syncthreads();
    const int lane = lane_id();
    const int tl = (int)threadIdx.x / G;   // the work-group's token, 0 .. 15
    const int64_t t = (int64_t)blockIdx.x * kHalfTokens + tl;
    const bool active = t < T;
    float v[VPL];
    uint32_t key[VPL];
    load_logits<VPL, VEC>(logits, t, active, E, lane % G, v, key);
    const int my_e = select_and_store<G, VPL>(v, key, active, t, E, k, topk_idx, topk_w);
    if (active && lane % G < k && (unsigned)my_e < (unsigned)E)
        atomicOr(&hmask[my_e], 1u << tl);
    __syncthreads();
    const int64_t word = blockIdx.x >> 1;
    const int half = (int)(blockIdx.x & 1);
    const bool clear_upper = half == 0 && blockIdx.x == gridDim.x - 1;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        uint16_t *p = half_masks + ((int64_t)e * nwords + word) * 2;
        p[half] = (uint16_t)hmask[e];
        if (clear_upper)
            p[1] = 0;
    }
}

// ---------------------------------------------------------------------------
// Group-limited ("node-limited") selection.  Handbook "NVSHMEM and DeepEP",
// "High-throughput mode": each node (here: a group of E/n_groups consecutive
// experts) is scored by the sum of its two best expert scores (logits), only
// the topk_groups best groups stay eligible (equal scores: the lower group),
// and the k experts are chosen among them.  Weights are unchanged: the full
// softmax over all E.
//
// One token per wave, or (large batches, at most 16 groups) one token per
// 16-lane group; lane l of a token holds experts l*VPL .. l*VPL+VPL-1.  A group's
// two best logits come from a "top-2 merge" reduction on order keys
// ((a1 >= a2) with (b1 >= b2) -> max(a1, b1), max(min(a1, b1), max(a2, b2)),
// the top two of the union), which commutes, so the result does not depend
// on the reduction order.  When a group is a power-of-two run of whole lanes
// (lanes_per_group = E/n_groups/VPL), every group is reduced at once by a
// butterfly inside its own lanes; otherwise groups are reduced one by one
// over the whole wave.  The score is the fp32 sum of the two values.

__device__ __forceinline__ void top2_merge(uint32_t &a1, uint32_t &a2, uint32_t b1, uint32_t b2)
{
    const uint32_t n2 = umax(a1 < b1 ? a1 : b1, umax(a2, b2));
    a1 = umax(a1, b1);
    a2 = n2;
}

template <int CTRL>
__device__ __forceinline__ void top2_dpp(uint32_t &a1, uint32_t &a2)
{
    top2_merge(a1, a2, dpp<CTRL>(a1), dpp<CTRL>(a2));
}

__device__ __forceinline__ void top2_xor(uint32_t &a1, uint32_t &a2, int m)
{
    top2_merge(a1, a2, (uint32_t)__shfl_xor((int)a1, m), (uint32_t)__shfl_xor((int)a2, m));
}

// Top two keys of a lane's eligible keys (a key of 0 is "none"), branch
// free: adding x to a multiset whose top two are (a1 >= a2) gives
// (max(a1, x), max(a2, min(a1, x))).  (An if/else chain here compiled to
// divergent branches and doubled the grouped router's time.)
template <int VPL>
__device__ __forceinline__ void lane_top2(const uint32_t (&key)[VPL], uint32_t mask_bits, uint32_t &a1, uint32_t &a2)
{
    a1 = 0u;
    a2 = 0u;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const uint32_t x = ((mask_bits >> i) & 1u) ? key[i] : 0u;
        a2 = umax(a2, a1 < x ? a1 : x);
        a1 = umax(a1, x);
    }
}

__device__ __forceinline__ uint32_t group_score_key(uint32_t t1, uint32_t t2)
{
    return order_key(key_value(t1) + key_value(t2));
}

// The token's topk_groups best groups as a bit set, from the score keys that
// lanes 0 .. n_groups-1 of its G lanes hold (the lowest group among equal
// scores): topk_groups rounds of a group max and a ballot.
template <int G>
__device__ __forceinline__ uint64_t pick_groups(uint32_t gkey, int topk_groups)
{
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    uint64_t kept = 0;
    for (int m = 0; m < topk_groups; ++m) {
        const uint32_t gm = group_max<G>(gkey);
        const uint64_t ball = __ballot(gkey == gm);
        const int g = __ffsll((unsigned long long)(G == kWave ? ball : (ball >> (grp * G)) & 0xFFFFull)) - 1;
        kept |= 1ull << g;
        if (gl == g)
            gkey = 0u;
    }
    return kept;
}

template <int G, int VPL, bool VEC, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void route_group_topk_kernel(const float *__restrict__ logits, int64_t T, int E,
                                                                  int k, int n_groups, int topk_groups,
                                                                  int lanes_per_group, int32_t *__restrict__ topk_idx,
                                                                  float *__restrict__ topk_w)
{
    static_assert(G == 16 || G == kWave, "16-lane groups or whole waves");
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = wave * (kWave / G) + grp;
    const bool active = t < T;
    float v[VPL];
    uint32_t key[VPL];
    load_logits<VPL, VEC>(logits, t, active, E, gl, v, key);
    const int gs = E / n_groups;
    uint32_t gkey = 0u;   // lane g < n_groups of the token: group g's score key (n_groups <= G)
    uint32_t tmax = 0u;   // the token's largest logit (key): the best group top-1
    uint64_t kept = 0;    // the token's kept groups
    if (ALIGNED) {
        // every group is a power-of-two run of L whole lanes: all groups at
        // once, by a butterfly inside their own lanes
        const int L = lanes_per_group;
        uint32_t a1, a2;
        lane_top2<VPL>(key, 0xFFFFu, a1, a2);
        if (L >= 2) top2_dpp<kDppQuadXor1>(a1, a2);
        if (L >= 4) top2_dpp<kDppQuadXor2>(a1, a2);
        if (L >= 8) top2_dpp<kDppHalfMirror>(a1, a2);
        if (L >= 16) top2_dpp<kDppMirror>(a1, a2);
        if (L >= 32) top2_xor(a1, a2, 16);
        if (L >= 64) top2_xor(a1, a2, 32);
        tmax = group_max<G>(a1);
        const uint32_t sk = group_score_key(a1, a2);
        const int src = grp * G + (gl < n_groups ? gl * L : 0);
        const uint32_t g_sk = (uint32_t)__shfl((int)sk, src);
        gkey = gl < n_groups ? g_sk : 0u;
    } else {
        // group of each of the lane's experts (n_groups: none).  The experts
        // are consecutive, so one division gives the first group and offset
        // and the rest follow by counting.
        int eg[VPL];
        {
            const int e0 = gl * VPL;
            int g = e0 / gs;
            int r = e0 - g * gs;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                eg[i] = e0 + i < E ? g : n_groups;
                if (++r == gs) {
                    r = 0;
                    ++g;
                }
            }
        }
        for (int g = 0; g < n_groups; ++g) {
            uint32_t bits = 0u;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (eg[i] == g)
                    bits |= 1u << i;
            uint32_t a1, a2;
            lane_top2<VPL>(key, bits, a1, a2);
            top2_dpp<kDppQuadXor1>(a1, a2);
            top2_dpp<kDppQuadXor2>(a1, a2);
            top2_dpp<kDppHalfMirror>(a1, a2);
            top2_dpp<kDppMirror>(a1, a2);
            uint32_t r1 = a1, r2 = a2;      // 16-lane groups: every lane of the row holds the result
            if (G == kWave) {
                r1 = (uint32_t)lane_value((int)a1, 0);
                r2 = (uint32_t)lane_value((int)a2, 0);
                top2_merge(r1, r2, (uint32_t)lane_value((int)a1, 16), (uint32_t)lane_value((int)a2, 16));
                top2_merge(r1, r2, (uint32_t)lane_value((int)a1, 32), (uint32_t)lane_value((int)a2, 32));
                top2_merge(r1, r2, (uint32_t)lane_value((int)a1, 48), (uint32_t)lane_value((int)a2, 48));
            }
            tmax = umax(tmax, r1);
            if (gl == g)
                gkey = group_score_key(r1, r2);
        }
        kept = pick_groups<G>(gkey, topk_groups);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (eg[i] < n_groups && !((kept >> eg[i]) & 1ull))
                key[i] = 0u;
    }
    if (ALIGNED) {
        kept = pick_groups<G>(gkey, topk_groups);
        // a lane's experts all belong to group gl / L: one test per lane
        if (!((kept >> (gl / lanes_per_group)) & 1ull)) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                key[i] = 0u;
        }
    }
    select_and_store<G, VPL>(v, key, active, t, E, k, topk_idx, topk_w, tmax);
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

template <int G, int VPL>
hipError_t launch_grouped(const float *logits, int64_t T, int E, int k, int n_groups, int topk_groups, int32_t *idx,
                          float *w, hipStream_t s)
{
    constexpr int64_t tokens_per_block = (int64_t)kWavesPerBlock * (kWave / G);
    const int64_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    const int gs = E / n_groups;
    int lpg = 0;  // lanes per group when every group is a power-of-two run of whole lanes
    if (gs % VPL == 0) {
        const int L = gs / VPL;
        if ((L & (L - 1)) == 0 && L <= G)
            lpg = L;
    }
    const bool vec = VPL > 1 && E % VPL == 0 && (VPL == 2 ? ((uintptr_t)logits % 8 == 0)
                                                           : (E % 4 == 0 && (uintptr_t)logits % 16 == 0));
#define MOE_GROUPED(V, A)                                                                                         \
    hipLaunchKernelGGL((route_group_topk_kernel<G, VPL, V, A>), dim3((unsigned)blocks), dim3(kBlock), 0, s, logits, \
                       T, E, k, n_groups, topk_groups, lpg, idx, w)
    if (vec && lpg)
        MOE_GROUPED(true, true);
    else if (vec)
        MOE_GROUPED(true, false);
    else if (lpg)
        MOE_GROUPED(false, true);
    else
        MOE_GROUPED(false, false);
#undef MOE_GROUPED
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk_grouped(const float *logits, int64_t T, int E, int k, int n_groups, int topk_groups,
                                     int32_t *idx, float *w, hipStream_t s)
{
    // as for the plain router: four tokens per wave (16-lane groups) for
    // large batches, when every group's score fits a lane of the token
    if (T >= 6144 && n_groups <= 16 && E > 32 && E <= 256) {
        if (E <= 64) return launch_grouped<16, 4>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
        if (E <= 128) return launch_grouped<16, 8>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
        return launch_grouped<16, 16>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
    }
    if (E <= 64) return launch_grouped<kWave, 1>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
    if (E <= 128) return launch_grouped<kWave, 2>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
    if (E <= 256) return launch_grouped<kWave, 4>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
    if (E <= 512) return launch_grouped<kWave, 8>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
    return launch_grouped<kWave, 16>(logits, T, E, k, n_groups, topk_groups, idx, w, s);
}

hipError_t launch_route_topk_masks(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                                   uint32_t *masks, hipStream_t s)
{
    const int64_t nchunks = (T + kMaskChunk - 1) / kMaskChunk;
    hipLaunchKernelGGL(route_topk_mask_kernel, dim3((unsigned)nchunks), dim3(kBlock), 0, s, logits, T, E, k, idx, w,
                       masks, (int)nchunks);
    return hipGetLastError();
}

namespace {

// The router's lane layout for E experts and T tokens: G lanes per token,
// VPL logits per lane.  Every router launch takes it from here, so a token's
// weights (whose softmax sum runs over that layout) are the same bits
// whichever router kernel routes it.  Above 32 experts: four tokens per wave
// (16-lane groups) when there are enough tokens to fill the chip that way,
// else one token per wave (measured on MI355X at E = 256: 16-lane groups win
// from ~6000 tokens, 10.7 vs 14.1 us at 16384; one wave per token wins
// below, 3.5 vs 5.6 us at 128).
template <class F>
hipError_t with_router_shape(int64_t T, int E, F &&f)
{
    if (E <= 1) return f.template run<1, 1>();
    if (E <= 2) return f.template run<2, 1>();
    if (E <= 4) return f.template run<4, 1>();
    if (E <= 8) return f.template run<8, 1>();
    if (E <= 16) return f.template run<16, 1>();
    if (E <= 32) return f.template run<32, 1>();
    const bool wide = T >= 6144;
    if (E <= 64) return wide ? f.template run<16, 4>() : f.template run<64, 1>();
    if (E <= 128) return wide ? f.template run<16, 8>() : f.template run<64, 2>();
    if (E <= 256) return wide ? f.template run<16, 16>() : f.template run<64, 4>();
    if (E <= 512) return f.template run<64, 8>();
    return f.template run<64, 16>();
}

struct PlainRouter {
    const float *logits; int64_t T; int E, k; int32_t *idx; float *w; hipStream_t s;
    template <int G, int VPL>
    hipError_t run() { return launch<G, VPL>(logits, T, E, k, idx, w, s); }
};

struct HalfMaskRouter {
    const float *logits; int64_t T; int E, k; int32_t *idx; float *w; uint16_t *half_masks; hipStream_t s;
    template <int G, int VPL>
    hipError_t run()
    {
        if constexpr (G < 16) {   // E <= 8 has its own word-per-work-group kernel
            return hipErrorInvalidValue;
        } else {
            return launch_half<G, VPL>();
        }
    }
    template <int G, int VPL>
    hipError_t launch_half()
    {
        const int64_t blocks = (T + kHalfTokens - 1) / kHalfTokens;
        const int nwords = (int)((T + kMaskChunk - 1) / kMaskChunk);
        const bool vec = VPL > 1 && E % VPL == 0 && (VPL == 2 ? ((uintptr_t)logits % 8 == 0)
                                                               : (E % 4 == 0 && (uintptr_t)logits % 16 == 0));
        const dim3 grid((unsigned)blocks), block(kHalfTokens * G);
        const size_t lds = (size_t)E * 4;
        if (vec)
            hipLaunchKernelGGL((route_topk_half_mask_kernel<G, VPL, true>), grid, block, lds, s, logits, T, E, k,
                               idx, w, half_masks, nwords);
        else
            hipLaunchKernelGGL((route_topk_half_mask_kernel<G, VPL, false>), grid, block, lds, s, logits, T, E, k,
                               idx, w, half_masks, nwords);
        return hipGetLastError();
    }
};

}  // namespace

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                             hipStream_t s)
{
    return with_router_shape(T, E, PlainRouter{logits, T, E, k, idx, w, s});
}

hipError_t launch_route_topk_half_masks(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                                        uint32_t *masks, hipStream_t s)
{
    if (E <= 8)
        return hipErrorInvalidValue;
    return with_router_shape(T, E, HalfMaskRouter{logits, T, E, k, idx, w, (uint16_t *)masks, s});
}

}  // namespace moe
