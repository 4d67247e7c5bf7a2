// fp8_e4m3.hpp -- the E4M3 block encoding shared by dispatch's fp8 rows and
// the fp8 output of the fused combine epilogue (gfx950).
//
// AI-infra handbook, "NVSHMEM and DeepEP", "High-throughput mode":
// activations travel as FP8 with one fp32 scale per 128 elements.  Per
// block: sc = amax / 448 (IEEE division; 1 for an all-zero block) and each
// code is the OCP E4M3 encoding, rounded to nearest even and saturating at
// 448, of the IEEE quotient x / sc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// x / sc for one bf16 value, bit-identical to the IEEE division x / sc.
// With r = 1/sc (one IEEE division per scale block), q0 = x*r is within an
// ulp or so of the quotient; the residual x - q0*sc is exact in an FMA and
// one correction step q0 + res*r rounds to the IEEE quotient (Markstein's
// division scheme).  The residual underflows for tiny values, so |x| or sc
// below 2^-100 need the IEEE division itself (fast_ok); copysign keeps the
// sign of a zero quotient.  Checked bit for bit against the IEEE E4M3 codes
// for every bf16 x with |x| <= amax and every bf16 amax.
__device__ __forceinline__ float divide_fast(float x, float sc, float r)
{
    const float q0 = x * r;
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, sc, x), r, q0), x);
}
__device__ __forceinline__ bool fast_ok(float x) { return __builtin_fabsf(x) >= 0x1p-100f || x == 0.0f; }

// q[i] = x[i] / sc for N values: the fast quotient when every value (and the
// scale) allows it, else the IEEE division for all N -- one branch per N
// values instead of one per value; both give the IEEE quotient.
template <int N>
__device__ __forceinline__ void divide_all(const float *x, float sc, float *q)
{
    const float r = 1.0f / sc;
    bool ok = sc >= 0x1p-100f;
#pragma unroll
    for (int i = 0; i < N; ++i)
        ok &= fast_ok(x[i]);   // no short-circuit: one branch in all
    if (ok) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            q[i] = divide_fast(x[i], sc, r);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            q[i] = x[i] / sc;
    }
}

// Four quotients -> four OCP E4M3 codes in one word.  v_cvt_pk_fp8_f32
// rounds to nearest even; the clamp to +-448 makes it saturate (a magnitude
// above 448 becomes 448), matching the E4M3 encoding the codes are defined
// by on every fp32 input of magnitude <= 464 (checked exhaustively).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 16 bf16 values -> 16 E4M3 codes of x / sc.
__device__ __forceinline__ u32x4 quantize16(const float *f, float sc)
{
    float q[16];
    divide_all<16>(f, sc, q);
    return (u32x4){e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]), e4m3x4(q[8], q[9], q[10], q[11]),
                   e4m3x4(q[12], q[13], q[14], q[15])};
}

// 8 bf16 values -> 8 E4M3 codes of x / sc (two words, element 0 in the
// lowest byte).
__device__ __forceinline__ u32x2 quantize8(const float *f, float sc)
{
    float q[8];
    divide_all<8>(f, sc, q);
    return (u32x2){e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
}

// Largest v over aligned groups of G (8 or 16) lanes, in every lane of the
// group: two quad permutes (lane xor 1, xor 2), the half-row mirror (lane i
// <- 7 - i within 8) and for 16 the row mirror (i <- 15 - i).  DPP moves
// stay inside a 16-lane row, so a group only reads its own lanes, and the
// maximum is exact in any order.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int G>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    v = fmaxf(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_move<0x141>(v));   // row_half_mirror
    if (G == 16)
        v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
    return v;
}

// The block scale of a 128-element block whose largest magnitude is amax.
__device__ __forceinline__ float block_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

}  // namespace moe
