// device_common.hpp -- small gfx950 helpers shared by the library's kernels.
//
// Wave64 throughout: every kernel is written for 64-lane wavefronts and
// 256-thread work-groups (4 waves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// A launch holds at most 2^32 - 1 work-items along x (the dispatch packet's
// grid size is 32-bit); launchers check their grid against it.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t blocks, int block_size) { return blocks * block_size <= kMaxGridItems; }

// Lane id within the wavefront.
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Make a value provably wave-uniform so the compiler keeps it in an SGPR
// and uses scalar loads for addresses derived from it.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Value of lane `l` (l wave-uniform) as a scalar.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_value(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// bf16 pair in a 32-bit word -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (lo in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32 with both operands (two scalar casts compile
// to two conversions plus a shift and an OR).
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

}  // namespace moe
