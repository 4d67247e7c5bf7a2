// dispatch.hip -- per-expert counts, fixed-slot assignment and row packing
// (gfx950).
//
// Handbook "NVSHMEM and DeepEP", "Why MoE's all-to-all is hard": after
// routing, tokens are sorted by destination and counted per destination.
// Its "Low-latency mode": each expert owns a fixed number of slots so every
// token's write address is known on the device, with no host round trip.
// pplx blog, Dispatch: tokens land contiguously per expert for the grouped
// GEMM and each token's source index is kept for combine.  Handbook
// "High-throughput mode": FP8 dispatch with one scale per 128 elements.
//
// Slot order inside an expert is ascending source token.  The rank of
// (t, j) among the tokens routed to e is computed without order-dependent
// atomics, so the result is deterministic:
//   K1 count:  one work-group per chunk of 256 tokens builds, in LDS, a
//              256-bit membership mask per expert (atomic OR, which commutes),
//              then writes the chunk's per-expert histogram and each pair's
//              rank inside the chunk (popcount of the mask below its bit).
//   K2 scan:   one wave per expert turns the chunk histograms into exclusive
//              per-chunk offsets (wave prefix sums) and the true total count.
//   K3 pack:   one wave per (token, column segment) finishes the slot
//              (offset + rank, dropped when >= capacity), records token_slot
//              and recv_src, loads the row once in 16-byte vectors and stores
//              it to each of its k slots -- bf16 bit copies, or E4M3 codes
//              with per-128 fp32 scales.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kChunk = 256;          // tokens per K1 work-group (one bit each)
constexpr int kMaskWords = kChunk / 32;

__global__ __launch_bounds__(kBlock) void dispatch_count_kernel(const int32_t *__restrict__ topk_idx, int64_t T,
                                                                int E, int k, int nchunks,
                                                                int32_t *__restrict__ chunk_counts,
                                                                int32_t *__restrict__ local_rank)
{
    extern __shared__ uint32_t mask[];  // [E][kMaskWords]
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    for (int i = tid; i < E * kMaskWords; i += kBlock)
        mask[i] = 0u;
    __syncthreads();

    const int64_t t = (int64_t)c * kChunk + tid;
    const int word = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[t * k + j];
            if ((unsigned)e < (unsigned)E)
                atomicOr(&mask[e * kMaskWords + word], bit);
        }
    }
    __syncthreads();

    for (int e = tid; e < E; e += kBlock) {
        int n = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w)
            n += __popc(mask[e * kMaskWords + w]);
        chunk_counts[(int64_t)e * nchunks + c] = n;
    }

    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[t * k + j];
            int r = -1;
            if ((unsigned)e < (unsigned)E) {
                r = __popc(mask[e * kMaskWords + word] & (bit - 1u));
                for (int w = 0; w < word; ++w)
                    r += __popc(mask[e * kMaskWords + w]);
            }
            local_rank[t * k + j] = r;
        }
    }
}

// chunk_counts[e][c] -> exclusive prefix over c (in place); total -> counts[e].
__global__ __launch_bounds__(kBlock) void dispatch_scan_kernel(int32_t *__restrict__ chunk_counts, int E,
                                                               int nchunks, int32_t *__restrict__ expert_counts)
{
    const int lane = lane_id();
    const int e = uniform(blockIdx.x * kWavesPerBlock + (int)(threadIdx.x / kWave));
    if (e >= E)
        return;
    int32_t *row = chunk_counts + (int64_t)e * nchunks;
    int carry = 0;
    for (int base = 0; base < nchunks; base += kWave) {
        const int i = base + lane;
        const int v = i < nchunks ? row[i] : 0;
        int x = v;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o)
                x += y;
        }
        if (i < nchunks)
            row[i] = carry + x - v;
        carry += __shfl(x, kWave - 1);
    }
    if (lane == 0)
        expert_counts[e] = carry;
}

// Slot of pair (t, lane) for lanes < k, else -1.  Wave 0 of a token's
// segments also records token_slot and recv_src.
__device__ __forceinline__ int finish_slot(const int32_t *__restrict__ topk_idx,
                                           const int32_t *__restrict__ local_rank,
                                           const int32_t *__restrict__ chunk_base, int64_t t, int E, int k,
                                           int C, int nchunks, bool record, int32_t *__restrict__ token_slot,
                                           int32_t *__restrict__ recv_src)
{
    const int lane = lane_id();
    int slot = -1;
    if (lane < k) {
        const int e = topk_idx[t * k + lane];
        const int r = local_rank[t * k + lane];
        if ((unsigned)e < (unsigned)E && r >= 0) {
            const int64_t rr = (int64_t)chunk_base[(int64_t)e * nchunks + t / kChunk] + r;
            if (rr < C)
                slot = (int)((int64_t)e * C + rr);
        }
        if (record) {
            token_slot[t * k + lane] = slot;
            if (slot >= 0)
                recv_src[slot] = (int32_t)t;
        }
    }
    return slot;
}

constexpr int kBatch = 2;  // 16-byte vectors per lane in flight per store round

// bf16 rows: one wave per (token, segment); lane owns 16-byte vectors
// seg*vpl*64 + i*64 + lane, i < vpl.
__global__ __launch_bounds__(kBlock) void dispatch_pack_bf16_kernel(
    const uint4 *__restrict__ x, int64_t T, int nvec, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ local_rank, const int32_t *__restrict__ chunk_base, int E, int k, int C,
    int nchunks, int vpl, int segs, int32_t *__restrict__ token_slot, int32_t *__restrict__ recv_src,
    uint4 *__restrict__ recv_x)
{
    const int lane = lane_id();
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;
    const int slot = finish_slot(topk_idx, local_rank, chunk_base, t, E, k, C, nchunks, seg == 0, token_slot,
                                 recv_src);
    const uint4 *src = x + t * nvec;
    const int v0 = seg * vpl * kWave + lane;
    for (int i0 = 0; i0 < vpl; i0 += kBatch) {
        uint4 buf[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int v = v0 + (i0 + b) * kWave;
            if (i0 + b < vpl && v < nvec)
                buf[b] = src[v];
        }
        for (int j = 0; j < k; ++j) {
            const int s = lane_value(slot, j);
            if (s < 0)
                continue;
            uint4 *dst = recv_x + (int64_t)s * nvec;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int v = v0 + (i0 + b) * kWave;
                if (i0 + b < vpl && v < nvec)
                    dst[v] = buf[b];
            }
        }
    }
}

// OCP E4M3 encode, round to nearest even, saturating at +-448.  Works on
// the float's bit pattern: the 23-bit mantissa is rounded to 3 bits by
// adding half-minus-one plus the kept LSB; the exponent is re-biased from
// 127 to 7.  Magnitudes below 2^-6 are counted in units of 2^-9 (exact
// power-of-two scaling, then round-half-even to an integer).
__device__ __forceinline__ uint32_t e4m3_from_float(float q)
{
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;                                   // NaN
    } else if (a >= 0x43E00000u) {
        code = 0x7Eu;                                   // |q| >= 448 (and inf): saturate
    } else if (a < 0x3C800000u) {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // subnormal: units of 2^-9
    } else {
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;       // (exp << 3 | m3), rounded
        code = r - (120u << 3);                         // exponent bias 127 -> 7
        code = code > 0x7Eu ? 0x7Eu : code;
    }
    return sign | code;
}

// fp8 rows: lane owns 16 consecutive elements (two 16-byte bf16 loads, one
// 16-byte code store); 8 lanes form one 128-element scale block.
__global__ __launch_bounds__(kBlock) void dispatch_pack_fp8_kernel(
    const uint4 *__restrict__ x, int64_t T, int nvec16, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ local_rank, const int32_t *__restrict__ chunk_base, int E, int k, int C,
    int nchunks, int vpl, int segs, int32_t *__restrict__ token_slot, int32_t *__restrict__ recv_src,
    uint4 *__restrict__ recv_x, float *__restrict__ recv_scales)
{
    const int lane = lane_id();
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    if (t >= T)
        return;
    const int slot = finish_slot(topk_idx, local_rank, chunk_base, t, E, k, C, nchunks, seg == 0, token_slot,
                                 recv_src);
    const int nblk = nvec16 / 8;  // scale blocks per row
    const uint4 *src = x + t * (int64_t)nvec16 * 2;
    const int v0 = seg * vpl * kWave + lane;
    for (int i = 0; i < vpl; ++i) {
        const int v = v0 + i * kWave;      // 16-element group; the 8 lanes of a block share validity
        const bool ok = v < nvec16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
        if (ok) {
            lo = src[2 * v];
            hi = src[2 * v + 1];
        }
        float f[16];
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            f[2 * q] = bf16_lo(w[q]);
            f[2 * q + 1] = bf16_hi(w[q]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            amax = fmaxf(amax, fabsf(f[q]));
#pragma unroll
        for (int o = 1; o < 8; o <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o));
        const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
        uint32_t packed[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            packed[q] = e4m3_from_float(f[4 * q] / sc) | (e4m3_from_float(f[4 * q + 1] / sc) << 8) |
                        (e4m3_from_float(f[4 * q + 2] / sc) << 16) | (e4m3_from_float(f[4 * q + 3] / sc) << 24);
        }
        const uint4 codes = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        if (!ok)
            continue;
        for (int j = 0; j < k; ++j) {
            const int s = lane_value(slot, j);
            if (s < 0)
                continue;
            recv_x[(int64_t)s * nvec16 + v] = codes;
            if ((lane & 7) == 0)
                recv_scales[(int64_t)s * nblk + v / 8] = sc;
        }
    }
}

// Split each row into `segs` segments of `vpl` vectors per lane so that at
// least ~min_waves waves are in flight.
void split_rows(int64_t T, int nvec, int64_t min_waves, int *vpl, int *segs)
{
    const int max_segs = (nvec + kWave - 1) / kWave;
    int64_t want = T > 0 ? (min_waves + T - 1) / T : 1;
    int s = (int)(want < 1 ? 1 : (want > max_segs ? max_segs : want));
    int v = (nvec + s * kWave - 1) / (s * kWave);
    s = (nvec + v * kWave - 1) / (v * kWave);
    *vpl = v;
    *segs = s;
}

}  // namespace

size_t dispatch_workspace_bytes(int64_t T, int E, int k)
{
    const int64_t nchunks = (T + kChunk - 1) / kChunk;
    const int64_t a = ((int64_t)E * nchunks * 4 + 255) / 256 * 256;
    const int64_t b = (T * k * 4 + 255) / 256 * 256;
    return (size_t)(a + b);
}

hipError_t launch_dispatch(const uint16_t *x, int64_t T, int H, const int32_t *topk_idx, int E, int k, int C,
                           int dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                           int32_t *expert_counts, int32_t *token_slot, void *workspace, hipStream_t s)
{
    const int nchunks = (int)((T + kChunk - 1) / kChunk);
    int32_t *chunk_counts = (int32_t *)workspace;
    int32_t *local_rank =
        (int32_t *)((char *)workspace + ((int64_t)E * nchunks * 4 + 255) / 256 * 256);

    if (nchunks > 0) {
        hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kBlock), (size_t)E * kMaskWords * 4, s,
                           topk_idx, T, E, k, nchunks, chunk_counts, local_rank);
    }
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3((E + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, s,
                       chunk_counts, E, nchunks, expert_counts);
    if (T == 0)
        return hipGetLastError();

    int vpl, segs;
    if (dtype == 0) {
        const int nvec = H / 8;
        split_rows(T, nvec, 2048, &vpl, &segs);
        const int64_t tasks = T * segs;
        const int64_t blocks = (tasks + kWavesPerBlock - 1) / kWavesPerBlock;
        hipLaunchKernelGGL(dispatch_pack_bf16_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           (const uint4 *)x, T, nvec, topk_idx, local_rank, chunk_counts, E, k, C, nchunks, vpl,
                           segs, token_slot, recv_src, (uint4 *)recv_x);
    } else {
        const int nvec16 = H / 16;
        split_rows(T, nvec16, 2048, &vpl, &segs);
        const int64_t tasks = T * segs;
        const int64_t blocks = (tasks + kWavesPerBlock - 1) / kWavesPerBlock;
        hipLaunchKernelGGL(dispatch_pack_fp8_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           (const uint4 *)x, T, nvec16, topk_idx, local_rank, chunk_counts, E, k, C, nchunks, vpl,
                           segs, token_slot, recv_src, (uint4 *)recv_x, recv_scales);
    }
    return hipGetLastError();
}

}  // namespace moe
