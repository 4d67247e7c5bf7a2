// bench_floor.hip -- copy kernels that move exactly the bytes of the dispatch
// pack and of combine, for the benchmark's floor comparison (bench.py
// --floor).  Not part of libmoe_route.so and not on the product path.
//
// Each kernel keeps the memory pattern of the kernel it stands beside --
// the same rows read and written at the same addresses, one wave per
// (token, row segment), every load of a lane issued before its stores,
// 16-byte vectors, non-temporal stores -- and drops everything else: no slot
// computation (the slots come from a finished dispatch), no quantisation,
// no floating point.  If the library's kernel runs as fast as its copy, the
// byte pattern, not the arithmetic, sets its time.
//
//   floor_scatter_rows  pack's pattern: each token's source row (2H bytes)
//                       read once, then written to each of its k slots: the
//                       whole row (bf16), or H bytes of it plus H/32 bytes
//                       to a second array (fp8 codes + per-128 fp32 scales)
//   floor_gather_rows   combine's pattern: each token's k rows (2H bytes
//                       each) and k weights read, one row of 2H bytes written
//   floor_scatter_writes  pack's stores alone: floor_scatter_rows with the
//                       source reads left out (each vector written is made
//                       from its token and position), to split pack's time
//                       between its writes and the reads mixed into them
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// bf16 rows: a lane copies VPL vectors of its segment to each slot.
template <int VPL, bool READ>
__global__ __launch_bounds__(kBlock) void scatter_bf16(const u32x4 *__restrict__ src, int64_t T, int nvec,
                                                       const int32_t *__restrict__ slot, int k, int segs,
                                                       u32x4 *__restrict__ dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;
    const int v0 = seg * VPL * kWave + lane;
    u32x4 buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v0 + i * kWave;
        if (READ)
            buf[i] = v < nvec ? src[t * nvec + v] : (u32x4){0, 0, 0, 0};
        else
            buf[i] = (u32x4){(uint32_t)t, (uint32_t)v, ~(uint32_t)t, ~(uint32_t)v};
    }
    int my = lane < k ? slot[t * k + lane] : -1;
    for (int j = 0; j < k; ++j) {
        const int s = __builtin_amdgcn_readlane(my, j);
        if (s < 0)
            continue;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave;
            if (v < nvec)
                __builtin_nontemporal_store(buf[i], dst + (int64_t)s * nvec + v);
        }
    }
}

// fp8 rows: a lane reads two 16-element groups (2 x 32 bytes) and writes
// 16 bytes per group to each slot's code row; the first lane of every 8
// groups (one 128-element block) also writes 4 bytes to the scale row.
template <bool READ>
__global__ __launch_bounds__(kBlock) void scatter_fp8(const u32x4 *__restrict__ src, int64_t T, int ngrp,
                                                      const int32_t *__restrict__ slot, int k, int segs,
                                                      u32x4 *__restrict__ codes, uint32_t *__restrict__ scales)
{
    constexpr int VPL = 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;
    const int g0 = seg * VPL * kWave + lane;
    u32x4 lo[VPL], hi[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int g = g0 + i * kWave;
        if (READ) {
            lo[i] = g < ngrp ? src[(t * ngrp + g) * 2] : (u32x4){0, 0, 0, 0};
            hi[i] = g < ngrp ? src[(t * ngrp + g) * 2 + 1] : (u32x4){0, 0, 0, 0};
        } else {   // lo ^ hi = {t, g, ~t, ~g}; lo[0] = t
            lo[i] = (u32x4){(uint32_t)t, 0u, 0u, 0u};
            hi[i] = (u32x4){0u, (uint32_t)g, ~(uint32_t)t, ~(uint32_t)g};
        }
    }
    int my = lane < k ? slot[t * k + lane] : -1;
    const int nblk = ngrp / 8;
    for (int j = 0; j < k; ++j) {
        const int s = __builtin_amdgcn_readlane(my, j);
        if (s < 0)
            continue;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int g = g0 + i * kWave;
            if (g >= ngrp)
                continue;
            __builtin_nontemporal_store(lo[i] ^ hi[i], codes + (int64_t)s * ngrp + g);
            if ((g & 7) == 0)
                __builtin_nontemporal_store(lo[i][0], scales + (int64_t)s * nblk + g / 8);
        }
    }
}

// combine's pattern: a lane loads VPL vectors of each of the K rows, then
// writes their XOR.
template <int K, int VPL>
__global__ __launch_bounds__(kBlock) void gather(const u32x4 *__restrict__ y, int64_t nrows, int nvec,
                                                 const int32_t *__restrict__ slot, const uint32_t *__restrict__ w,
                                                 int64_t T, int segs, u32x4 *__restrict__ out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;
    int my = -1;
    uint32_t myw = 0;
    if (lane < K) {
        const int s = slot[t * K + lane];
        my = (s >= 0 && s < nrows) ? s : -1;
        myw = w[t * K + lane];
    }
    int rows[K];
    uint32_t wb = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        rows[j] = __builtin_amdgcn_readlane(my, j);
        wb ^= (uint32_t)__builtin_amdgcn_readlane((int)myw, j);
    }
    const int v0 = seg * VPL * kWave + lane;
    u32x4 buf[K][VPL];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave;
            buf[j][i] = (rows[j] >= 0 && v < nvec) ? __builtin_nontemporal_load(y + (int64_t)rows[j] * nvec + v)
                                                   : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v0 + i * kWave;
        if (v >= nvec)
            continue;
        u32x4 acc = {wb, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < K; ++j)
            acc ^= buf[j][i];
        __builtin_nontemporal_store(acc, out + t * nvec + v);
    }
}

int64_t blocks_for(int64_t T, int segs) { return (T * segs + kWaves - 1) / kWaves; }

template <int K>
hipError_t gather_k(const void *y, int64_t nrows, int nvec, const int32_t *slot, const uint32_t *w, int64_t T,
                    void *out, hipStream_t s)
{
    constexpr int VPL = K <= 4 ? 8 : (K <= 8 ? 4 : 2);
    const int segs = (nvec + VPL * kWave - 1) / (VPL * kWave);
    hipLaunchKernelGGL((gather<K, VPL>), dim3((unsigned)blocks_for(T, segs)), dim3(kBlock), 0, s,
                       (const u32x4 *)y, nrows, nvec, slot, w, T, segs, (u32x4 *)out);
    return hipGetLastError();
}

template <bool READ>
int scatter(const void *x, int64_t T, int32_t H, int32_t fp8, const int32_t *token_slot, int32_t k, void *recv_x,
            void *recv_scales, hipStream_t s)
{
    if (fp8) {
        const int ngrp = H / 16;
        const int segs = (ngrp + 2 * kWave - 1) / (2 * kWave);
        hipLaunchKernelGGL(scatter_fp8<READ>, dim3((unsigned)blocks_for(T, segs)), dim3(kBlock), 0, s,
                           (const u32x4 *)x, T, ngrp, token_slot, k, segs, (u32x4 *)recv_x, (uint32_t *)recv_scales);
        return (int)hipGetLastError();
    }
    const int nvec = H / 8;
    int vpl = k >= 8 ? 1 : 8 / k;
    vpl = vpl >= 8 ? 8 : (vpl >= 4 ? 4 : (vpl >= 2 ? 2 : 1));
    const int segs = (nvec + vpl * kWave - 1) / (vpl * kWave);
    const dim3 grid((unsigned)blocks_for(T, segs));
    const u32x4 *src = (const u32x4 *)x;
    u32x4 *dst = (u32x4 *)recv_x;
    switch (vpl) {
    case 1: hipLaunchKernelGGL((scatter_bf16<1, READ>), grid, dim3(kBlock), 0, s, src, T, nvec, token_slot, k, segs, dst); break;
    case 2: hipLaunchKernelGGL((scatter_bf16<2, READ>), grid, dim3(kBlock), 0, s, src, T, nvec, token_slot, k, segs, dst); break;
    case 4: hipLaunchKernelGGL((scatter_bf16<4, READ>), grid, dim3(kBlock), 0, s, src, T, nvec, token_slot, k, segs, dst); break;
    default: hipLaunchKernelGGL((scatter_bf16<8, READ>), grid, dim3(kBlock), 0, s, src, T, nvec, token_slot, k, segs, dst); break;
    }
    return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// Returns 0, -1 for a bad argument, or the HIP error of the launch.
__attribute__((visibility("default"))) int floor_scatter_rows(const void *x, int64_t T, int32_t H, int32_t fp8,
                                                               const int32_t *token_slot, int32_t k, void *recv_x,
                                                               void *recv_scales, hipStream_t s)
{
    if (T < 1 || k < 1 || k > 64 || H % (fp8 ? 128 : 8) != 0 || !x || !token_slot || !recv_x ||
        (fp8 && !recv_scales))
        return -1;
    return scatter<true>(x, T, H, fp8, token_slot, k, recv_x, recv_scales, s);
}

// floor_scatter_rows without the source: the same slots, launch shape and
// stores, with no loads of x.
__attribute__((visibility("default"))) int floor_scatter_writes(int64_t T, int32_t H, int32_t fp8,
                                                                 const int32_t *token_slot, int32_t k, void *recv_x,
                                                                 void *recv_scales, hipStream_t s)
{
    if (T < 1 || k < 1 || k > 64 || H % (fp8 ? 128 : 8) != 0 || !token_slot || !recv_x || (fp8 && !recv_scales))
        return -1;
    return scatter<false>(nullptr, T, H, fp8, token_slot, k, recv_x, recv_scales, s);
}

__attribute__((visibility("default"))) int floor_gather_rows(const void *y, int64_t nrows, int32_t H,
                                                              const int32_t *token_slot, const void *topk_w, int64_t T,
                                                              int32_t k, void *out, hipStream_t s)
{
    if (T < 1 || nrows < 1 || H % 8 != 0 || !y || !token_slot || !topk_w || !out)
        return -1;
    const int nvec = H / 8;
    const uint32_t *w = (const uint32_t *)topk_w;
    switch (k) {
#define FLOOR_K(K) \
    case K: return (int)gather_k<K>(y, nrows, nvec, token_slot, w, T, out, s);
    FLOOR_K(1) FLOOR_K(2) FLOOR_K(3) FLOOR_K(4) FLOOR_K(5) FLOOR_K(6) FLOOR_K(7) FLOOR_K(8)
    FLOOR_K(9) FLOOR_K(10) FLOOR_K(11) FLOOR_K(12) FLOOR_K(13) FLOOR_K(14) FLOOR_K(15) FLOOR_K(16)
#undef FLOOR_K
    default: return -1;
    }
}

}  // extern "C"
