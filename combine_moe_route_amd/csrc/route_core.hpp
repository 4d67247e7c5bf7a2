// route_core.hpp -- the router's selection and softmax device code (gfx950),
// shared by the router kernels and by the pack kernel that routes a small
// batch itself, so that every path produces the same bits.
//
// pplx blog "Efficient and portable mixture-of-experts communication",
// Introduction: the router yields a probability distribution over experts,
// the experts with the top-K scores are chosen and weighted by it.  The
// conventions (order keys, tie rule, fixed-order sums) are described in
// route_topk.hip.
#pragma once

#include "device_common.hpp"

namespace moe {
namespace route_core {

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within 16

// Under these patterns every lane reads a lane of its own row, so the
// bound_ctrl fill value (0) is never used; with it the compiler folds each
// move into the max or add that follows (one DPP-modified instruction).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
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

// Loads lane gl's VPL consecutive logits of token t (VEC: as one aligned
// vector) and their order keys; experts >= E and inactive tokens get key 0,
// which is below every real key.
template <int VPL, bool VEC>
__device__ __forceinline__ void load_logits(const float *__restrict__ logits, int64_t t, bool active, int E, int gl,
                                            float (&v)[VPL], uint32_t (&key)[VPL])
{
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
            key[i] = ok ? order_key(v[i]) : 0u;
        }
    }
}

// k selection rounds over the eligible keys (key 0 = not eligible), then the
// full softmax over every logit of the token (eligible or not) and the
// stores of token t's ids and weights.  max_key: order key of the token's
// largest logit when some experts were excluded; 0 when every expert was
// eligible, so that the first choice is the largest logit.
template <int G, int VPL>
__device__ __forceinline__ int select_and_store(const float (&v)[VPL], uint32_t (&key)[VPL], bool active, int64_t t,
                                                 int E, int k, int32_t *__restrict__ topk_idx,
                                                 float *__restrict__ topk_w, uint32_t max_key = 0u)
{
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
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
            e = VPL == 1 ? wl : wl * VPL + __shfl(bi, grp * G + wl);
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

    // the softmax's maximum is the largest logit of all; with every expert
    // eligible it is the first choice
    float s = 0.0f;
    const float mx = max_key ? key_value(max_key) : top;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (active && gl * VPL + i < E)
            s += expf(v[i] - mx);
    s = group_sum<G>(s);

    if (active && gl < k && topk_idx) {   // NULL outputs: choices only (uniform test)
        topk_idx[t * k + gl] = my_e;
        topk_w[t * k + gl] = expf(my_v - mx) / s;
    }
    return my_e;    // lane gl < k of an active token: its choice j = gl
}

}  // namespace route_core
}  // namespace moe
