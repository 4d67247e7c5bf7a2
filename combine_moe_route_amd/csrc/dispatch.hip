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
//   count:  one work-group per chunk of 256 tokens builds, in LDS, a 256-bit
//           membership mask per expert (atomic OR, which commutes), then
//           writes the chunk's per-expert histogram and each pair's rank
//           inside the chunk (popcount of the mask below its bit).
//   pack:   one wave per (token, row segment) requests all of its row
//           vectors, then works out the k slots:
//           offset = sum of the expert's counts in earlier chunks (an
//           exclusive prefix over a few L2-resident histogram words),
//           slot = e*C + offset + rank, dropped when >= C.  Segment 0
//           records token_slot and recv_src; then the row is stored to
//           each slot -- bf16 bit copies, or E4M3 codes with per-128 fp32
//           scales.  The first E waves also write the true totals.
//   scan:   past 256 chunks that prefix would grow with the batch, so one
//           work-group per expert first rewrites the expert's chunk counts
//           as exclusive prefixes (and writes its total); pack then reads
//           the prefix with one load.
// A batch of at most 256 tokens is a single chunk: then there is no count
// launch, and every pack work-group rebuilds the chunk's masks in LDS from
// ids it requests before the rows.  Up to 1024 tokens whose ids fit 32 per
// thread (and whose masks are at most 8192 words) are counted the same way.
// Route + dispatch in one call: the router already wrote one membership
// word per expert and 32-token chunk (for E > 8 as two 16-token halves, on
// batches past the in-pack limits while each pair's prefix stays a bounded
// number of word loads), and pack takes prefixes and ranks from their
// popcounts (no count launch either).
// Packed, count-sized layout (handbook "High-throughput mode": count first,
// then a receive buffer of exactly the needed size): between count and
// pack, one work-group sums each expert's chunk counts (or the popcounts of
// the router's words) and scans them into offsets[E+1]; a single chunk's
// pack work-groups scan their LDS counts, and with at most 2048 router words
// every pack work-group totals and scans them itself.  Pack then uses slot =
// offsets[e] + offset + rank, with no capacity and nothing dropped.
// Slot rows are written with non-temporal stores: each byte is written once
// per call.
#include "device_common.hpp"
#include "fp8_e4m3.hpp"
#include "kernels.hpp"
#include "route_core.hpp"

namespace moe {
namespace {

constexpr int kChunk = 256;          // tokens per count work-group (one mask bit each)
constexpr int kMaskWords = kChunk / 32;
// LDS membership masks are laid out [E][stride] with an odd stride (one word
// of padding): with a power-of-two stride, the lanes of one instruction that
// read or OR word w of different experts all hit a few LDS banks; an odd
// stride spreads them over every bank.
constexpr int kMaskStride = kMaskWords + 1;
constexpr int kMaskChunk = 32;       // tokens per router membership word
constexpr int kLocalTokens = 4 * kChunk;   // pack counts the batch itself up to this many tokens
constexpr int kMaxK = 16;                  // the largest k the library accepts (MOE_MAX_TOPK)

// Membership words per expert kept in LDS by the pack modes that count the
// batch themselves: one 256-token chunk's 8, or ceil(T/32) for larger batches.
__host__ __device__ constexpr int local_words(int64_t T)
{
    return T <= kChunk ? kMaskWords : (int)((T + 31) / 32);
}
__host__ __device__ constexpr int local_stride(int nw) { return nw | 1; }

// Sum of v over aligned groups of g lanes (g a power of two, 1 .. 64), in
// every lane of the group; every lane of the wave must be active.  Up to 16
// lanes the partial sums move by DPP inside a 16-lane row (lane xor 1,
// xor 2, then the half-row mirror i <- 7 - i and the row mirror
// i <- 15 - i, which pair each lane with one of the other half); wider
// groups add cross-row shuffles.  Integer sums are exact in any order.
template <int CTRL>
__device__ __forceinline__ int dpp_int(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int group_sum(int v, int g)
{
    if (g > 1)
        v += dpp_int<0xB1>(v);    // quad_perm [1,0,3,2]
    if (g > 2)
        v += dpp_int<0x4E>(v);    // quad_perm [2,3,0,1]
    if (g > 4)
        v += dpp_int<0x141>(v);   // row_half_mirror
    if (g > 8)
        v += dpp_int<0x140>(v);   // row_mirror
    if (g > 16)
        v += __shfl_xor(v, 16);
    if (g > 32)
        v += __shfl_xor(v, 32);
    return v;
}

// p / k for 0 <= p < 8192 and 1 <= k <= 16 as (p * ceil(2^17 / k)) >> 17:
// the multiplier overshoots 2^17 / k by less than 1, which adds less than
// p / 2^17 to p / k, and the fraction of p / k is at most (k - 1) / k, so
// the floor is unchanged while 8191 (k - 1) < 2^17 (p * mul < 2^30).
__host__ __device__ constexpr uint32_t small_div_mul(int k) { return (131072u + (uint32_t)k - 1u) / (uint32_t)k; }
__host__ __device__ constexpr int small_div(int p, uint32_t mul) { return (int)(((uint32_t)p * mul) >> 17); }
constexpr bool small_div_exact(int k)
{
    for (int p = 0; p < 8192; ++p)
        if (small_div(p, small_div_mul(k)) != p / k)
            return false;
    return true;
}
static_assert(small_div_exact(1) && small_div_exact(2) && small_div_exact(3) && small_div_exact(4) &&
              small_div_exact(5) && small_div_exact(6) && small_div_exact(7) && small_div_exact(8) &&
              small_div_exact(9) && small_div_exact(10) && small_div_exact(11) && small_div_exact(12) &&
              small_div_exact(13) && small_div_exact(14) && small_div_exact(15) && small_div_exact(16),
              "multiply-shift division is exact for every pair index of a local batch");

// Exclusive scan of the work-group's n <= 4*256 values in LDS (thread i owns
// values 4i .. 4i+3): out[i] = sum of in[0 .. i-1] for i < n, out[n] = total.
// out may be in: a thread reads its own values before the barrier and
// writes only those (and out[n]) after it.
__device__ __forceinline__ void block_exclusive_scan(const int32_t *in, int n, int32_t *out, int32_t *wave_sums)
{
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / kWave;
    int v[4];
    int own = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v[u] = 4 * tid + u < n ? in[4 * tid + u] : 0;
        own += v[u];
    }
    int incl = own;
    for (int o = 1; o < kWave; o <<= 1) {
        const int up = __shfl_up(incl, o);
        if (lane >= o)
            incl += up;
    }
    if (lane == kWave - 1)
        wave_sums[wv] = incl;
    __syncthreads();
    int run = incl - own;
    for (int w = 0; w < wv; ++w)
        run += wave_sums[w];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (4 * tid + u < n)
            out[4 * tid + u] = run;
        run += v[u];
        if (4 * tid + u == n - 1)
            out[n] = run;
    }
}

// The count kernel's LDS row per expert: the chunk's 8 membership words,
// then the exclusive prefix of their popcounts as 8 bytes in 2 words (each
// at most 7 * 32 = 224), then one word of padding so the stride is odd.
constexpr int kCountPrefix = kMaskWords;            // word offset of the prefix bytes
constexpr int kCountStride = kMaskWords + 2 + 1;    // 11

__global__ __launch_bounds__(kBlock) void dispatch_count_kernel(const int32_t *__restrict__ topk_idx, int64_t T,
                                                                int E, int k, int nchunks,
                                                                int32_t *__restrict__ chunk_counts,
                                                                int32_t *__restrict__ local_rank)
{
    extern __shared__ uint32_t mask[];  // [E][kCountStride]
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    for (int i = tid; i < E * kCountStride; i += kBlock)
        mask[i] = 0u;
    __syncthreads();

    const int64_t t = (int64_t)c * kChunk + tid;
    const int word = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);
    // The token's ids, loaded once.  Lanes walk their k choices starting at
    // different positions (j0 = lane mod k): with skewed routing a hot expert
    // tends to sit at the same position j for many tokens, and lanes of one
    // 32-token word ORing into the same LDS word in one instruction
    // serialise; rotated, such lanes mostly land in different instructions.
    int ids[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
        ids[j] = (t < T && j < k) ? topk_idx[t * k + j] : -1;
    const int j0 = tid % k;
    if (t < T) {
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) {
            if (jj >= k)
                break;
            int j = j0 + jj;
            j = j >= k ? j - k : j;
            int e = -1;
#pragma unroll
            for (int q = 0; q < kMaxK; ++q)
                e = q == j ? ids[q] : e;
            if ((unsigned)e < (unsigned)E)
                atomicOr(&mask[e * kCountStride + word], bit);
        }
    }
    __syncthreads();

    // per expert: the chunk's count, and the prefix of each word's popcount
    for (int e = tid; e < E; e += kBlock) {
        uint32_t *row = mask + e * kCountStride;
        uint32_t pre[2] = {0u, 0u};
        int n = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) {
            pre[w >> 2] |= (uint32_t)n << (8 * (w & 3));
            n += __popc(row[w]);
        }
        row[kCountPrefix] = pre[0];
        row[kCountPrefix + 1] = pre[1];
        chunk_counts[(int64_t)e * nchunks + c] = n;
    }
    __syncthreads();

    // rank of (t, j) in the chunk: earlier words' total + earlier bits of its own word
    if (t < T) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k)
                break;
            const int e = ids[j];
            int r = -1;
            if ((unsigned)e < (unsigned)E) {
                const uint32_t *row = mask + e * kCountStride;
                r = __popc(row[word] & (bit - 1u)) + (int)((row[kCountPrefix + (word >> 2)] >> (8 * (word & 3))) & 0xFFu);
            }
            local_rank[t * k + j] = r;
        }
    }
}

// T = 0: nothing routed, every count (or offset) is zero.
__global__ __launch_bounds__(kBlock) void dispatch_zero_counts_kernel(int32_t *__restrict__ expert_counts, int E)
{
    for (int e = blockIdx.x * kBlock + threadIdx.x; e < E; e += gridDim.x * kBlock)
        expert_counts[e] = 0;
}

// Beyond this many 256-token chunks the pack's per-pair prefix (a sum over
// every earlier chunk) would grow with the batch, so the chunk counts are
// scanned first.
constexpr int kScanChunks = 256;

// One work-group per expert e: chunk_counts[e][c] is replaced by the exclusive
// prefix sum over chunks 0 .. c-1 (in place, in pieces of 1024 chunks) and
// totals[e] (if given) receives the expert's total.
__global__ __launch_bounds__(kBlock) void dispatch_chunk_scan_kernel(int32_t *__restrict__ chunk_counts,
                                                                     int nchunks, int32_t *__restrict__ totals)
{
    __shared__ int32_t wave_sums[kWavesPerBlock];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / kWave;
    int32_t *row = chunk_counts + (int64_t)blockIdx.x * nchunks;
    int run = 0;   // total of the earlier pieces
    for (int c0 = 0; c0 < nchunks; c0 += 4 * kBlock) {
        int v[4];
        int own = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + 4 * tid + u;
            v[u] = c < nchunks ? row[c] : 0;
            own += v[u];
        }
        int incl = own;
        for (int o = 1; o < kWave; o <<= 1) {
            const int up = __shfl_up(incl, o);
            if (lane >= o)
                incl += up;
        }
        if (lane == kWave - 1)
            wave_sums[wv] = incl;
        __syncthreads();
        int base = run + incl - own;
        int piece = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) {
            base += w < wv ? wave_sums[w] : 0;
            piece += wave_sums[w];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + 4 * tid + u;
            if (c < nchunks)
                row[c] = base;
            base += v[u];
        }
        run += piece;
        __syncthreads();   // wave_sums is rewritten by the next piece
    }
    if (tid == 0 && totals)
        totals[blockIdx.x] = run;
}

constexpr int kScanBlock = 1024;                      // >= the largest E
constexpr int kScanWaves = kScanBlock / kWave;

// Packed layout: offsets[e] = sum of the counts of experts below e, and
// offsets[E] = the total, from the [E][nchunks] chunk histograms.  One
// work-group: `tpe` consecutive threads (a power of two <= 64) total one
// expert's row, each summing every tpe-th chunk with eight loads in flight,
// then a butterfly; then a work-group exclusive scan over the E totals (wave
// scans, then the wave sums).
// MASKS: the rows are the router's 32-token membership words (uint32), and
// an expert's total is the sum of their popcounts; otherwise the rows are
// the 256-token chunk histograms.
template <bool MASKS>
__global__ __launch_bounds__(kScanBlock) void dispatch_offsets_kernel(const int32_t *__restrict__ chunk_counts,
                                                                      int E, int nchunks,
                                                                      int32_t *__restrict__ offsets)
{
    __shared__ int32_t total[kScanBlock];
    __shared__ int32_t wave_sum[kScanWaves];
    const int lane = lane_id();
    const int wv = threadIdx.x / kWave;
    int tpe = kWave;
    while (tpe > 1 && tpe * E > kScanBlock)
        tpe >>= 1;
    const int per_pass = kScanBlock / tpe;
    const int sub = threadIdx.x % tpe;
    for (int e0 = 0; e0 < E; e0 += per_pass) {
        const int e = e0 + (int)threadIdx.x / tpe;
        int sum = 0;
        if (e < E) {
            const int32_t *row = chunk_counts + (int64_t)e * nchunks;
            for (int cc = sub; cc < nchunks; cc += 8 * tpe) {
                int part[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    part[u] = cc + u * tpe < nchunks ? row[cc + u * tpe] : 0;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    sum += MASKS ? __popc((uint32_t)part[u]) : part[u];
            }
        }
        for (int o = tpe / 2; o > 0; o >>= 1)
            sum += __shfl_xor(sum, o);
        if (sub == 0 && e < E)
            total[e] = sum;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    const int v = tid < E ? total[tid] : 0;
    int incl = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const int up = __shfl_up(incl, o);
        if (lane >= o)
            incl += up;
    }
    if (lane == kWave - 1)
        wave_sum[wv] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w)
        base += wave_sum[w];
    const int excl = base + incl - v;
    if (tid < E)
        offsets[tid] = excl;
    if (tid == E - 1)
        offsets[E] = excl + v;
}

// Streaming stores: every slot byte is written once per call and not read
// back by this call, so stores are non-temporal.  (Measured on MI355X: the
// row loads are faster as ordinary loads, the stores as non-temporal ones.)
__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(float *p, float v) { __builtin_nontemporal_store(v, p); }

// A batch of at most 256 tokens is one chunk: every pack work-group then
// rebuilds that chunk's membership masks from the ids itself (T*k ids, read
// from L2), so no count launch is needed; up to 1024 tokens are counted the
// same way, with ceil(T/32) words per expert (local_words).  The ids are requested before the
// row loads (local_ids_load): vector loads retire in order, so waiting for
// ids issued after the rows would wait for the rows too.  lds: [E][nw | 1] mask
// words, then for the packed layout [E+1] offsets (the exclusive scan of the
// popcounts).  The totals are published by the work-groups in turn (expert e
// by work-group e mod gridDim.x); work-group 0 publishes the offsets.  All
// threads must call both.
constexpr int kLocalIds = kChunk * 16 / kBlock;   // ids per thread: T*k <= 4096
constexpr int kLocalIdsWide = 2 * kLocalIds;      // the wide mode's: T*k <= 8192

// Whether pack counts the batch itself: one chunk, or up to 1024 tokens whose
// ids fit kLocalIdsWide per thread and whose masks are at most 8192 words
// (every work-group clears, fills and popcounts the masks, which past that
// costs more than the count launch it saves).  Past kLocalIds ids per thread
// the pack takes its wide mode (32 id registers per thread).
__host__ __device__ constexpr bool local_count(int64_t T, int E, int k)
{
    return T <= kChunk ||
           (T <= kLocalTokens && T * k <= (int64_t)kLocalIdsWide * kBlock && (int64_t)E * local_words(T) <= 8192);
}
__host__ __device__ constexpr bool local_ids_wide(int64_t T, int k) { return T * k > (int64_t)kLocalIds * kBlock; }

// The router's membership words replace the count launch while a pair's
// prefix (the popcounts of the earlier words of its expert) takes at most
// this many L2 loads per lane: for E > 8, and for E <= 8 with k > 4 (eight
// lanes or fewer per pair), 32; for E <= 8 with k <= 4, 64.  Measured in one
// process against route + count + pack: at 8 experts, top-8, the words win
// by 6% at 32 loads per lane and lose by 7-9% at 48 and 64; at top-2 they
// still win by 1-3% at 48 and 64 loads.
__host__ __device__ constexpr int mask_prefix_loads(int E, int k) { return E <= 8 && k <= 4 ? 64 : 32; }

// The single-chunk loads are issued unconditionally, from a clamped
// (in-bounds) index, and unwanted values discarded afterwards: a load under a
// branch makes the compiler wait for every outstanding load before the first
// use, which would make the counting wait for the rows.
template <int N>
__device__ __forceinline__ void local_ids_load(const int32_t *__restrict__ topk_idx, int n, int (&ids)[N])
{
#pragma unroll
    for (int q = 0; q < N; ++q) {
        const int p = (int)threadIdx.x + q * kBlock;
        const int v = topk_idx[p < n ? p : n - 1];
        ids[q] = p < n ? v : -1;
    }
}

// The chunk's per-expert totals from its complete LDS masks: each work-group
// writes those of the experts e with e mod gridDim.x == blockIdx.x (fixed
// slots; no work-group pays for all E), or every work-group scans them into
// loffs and work-group 0 writes the offsets (packed layout).  All threads
// call it.
__device__ __forceinline__ void local_totals(int E, int nw, int ns, bool packed, const uint32_t *lmask, int32_t *loffs,
                                             int32_t *wave_sums, int32_t *__restrict__ expert_counts,
                                             int32_t *__restrict__ expert_offsets)
{
    const int tid = threadIdx.x;
    if (!packed) {   // expert e's total is written by work-group e mod gridDim.x
        for (int e = (int)blockIdx.x + tid * (int)gridDim.x; e < E; e += kBlock * (int)gridDim.x) {
            int n = 0;
            for (int w = 0; w < nw; ++w)
                n += __popc(lmask[e * ns + w]);
            expert_counts[e] = n;
        }
        return;
    }
    for (int e = tid; e < E; e += kBlock) {
        int n = 0;
#pragma unroll
        for (int w = 0; w < nw; ++w)
            n += __popc(lmask[e * ns + w]);
        loffs[e] = n;
    }
    {
        __syncthreads();
        block_exclusive_scan(loffs, E, loffs, wave_sums);   // in place: each thread rewrites only what it read
        __syncthreads();
        if (blockIdx.x == 0)
            for (int e = tid; e <= E; e += kBlock)
                expert_offsets[e] = loffs[e];
    }
}

template <int N>
__device__ __forceinline__ void local_chunk_counts(const int (&ids)[N], int E, int k, int nw, int ns,
                                                   bool packed,
                                                   uint32_t *lmask, int32_t *loffs, int32_t *wave_sums,
                                                   int32_t *__restrict__ expert_counts,
                                                   int32_t *__restrict__ expert_offsets)
{
    const int tid = threadIdx.x;
    const uint32_t kmul = small_div_mul(k);
    for (int i = tid; i < E * ns; i += kBlock)
        lmask[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < N; ++q) {
        const int e = ids[q];   // pair p = tid + q*256 of token p / k; -1 past the end
        if ((unsigned)e < (unsigned)E) {
            const int tok = small_div(tid + q * kBlock, kmul);
            atomicOr(&lmask[e * ns + (tok >> 5)], 1u << (tok & 31));
        }
    }
    __syncthreads();
    local_totals(E, nw, ns, packed, lmask, loffs, wave_sums, expert_counts, expert_offsets);
}

// Route + dispatch of a batch of at most 256 tokens with E <= 8 in one
// launch: every pack work-group routes the whole batch itself -- 8-lane
// groups, 32 tokens per pass, the router's own selection and softmax code,
// so the choices and weights are those of moe_route_topk bit for bit --
// keeping the choices in LDS (ids and membership masks); work-group 0 also
// stores ids and weights, and the totals are spread as in local_totals.  A lane's logits for all passes are
// requested before the row loads, for the reason given at local_ids_load.
constexpr int kRoutePasses = kChunk / kMaskChunk;   // 8 passes of 32 tokens

// Pack kernel modes: slots from chunk histograms or router membership words
// (several chunks); a single chunk counted in LDS from the ids; a single
// chunk routed in LDS by every work-group.
constexpr int kPackChunks = 0;
constexpr int kPackLocalIds = 1;
constexpr int kPackLocalRoute = 2;
// Packed layout from router membership words (E <= 8, several chunks): every
// pack work-group totals the words itself and scans the totals into LDS
// offsets, in place of a separate one-work-group offsets launch.
constexpr int kPackMaskOffsets = 3;
constexpr int kOffWords = 8;   // membership words per thread in that mode: E * words <= 8 * 256
// Several chunks whose counts dispatch_chunk_scan_kernel has already turned
// into per-expert exclusive prefixes: one load per pair instead of a sum.
constexpr int kPackScanned = 4;
// A single batch counted in LDS as kPackLocalIds, with kLocalIdsWide ids per
// thread (4096 < T*k <= 8192).
constexpr int kPackLocalIdsWide = 5;
template <int MODE>
__host__ __device__ constexpr bool local_ids_mode() { return MODE == kPackLocalIds || MODE == kPackLocalIdsWide; }
template <int MODE>
__host__ __device__ constexpr int local_ids_count() { return MODE == kPackLocalIdsWide ? kLocalIdsWide : kLocalIds; }

// The membership words [E][nwords] as kOffWords words per thread, requested
// before the row loads from a clamped index (see local_ids_load); words past
// the end read as 0.
__device__ __forceinline__ void mask_words_load(const uint32_t *__restrict__ masks, int n, uint32_t (&w)[kOffWords])
{
#pragma unroll
    for (int q = 0; q < kOffWords; ++q) {
        const int p = (int)threadIdx.x + q * kBlock;
        const uint32_t v = masks[p < n ? p : n - 1];
        w[q] = p < n ? v : 0u;
    }
}

// Popcounts of those words, taken right after the row loads are requested
// and before any branch, so that the compiler waits for the words alone.
__device__ __forceinline__ void mask_words_count(uint32_t (&w)[kOffWords])
{
#pragma unroll
    for (int q = 0; q < kOffWords; ++q)
        w[q] = __popc(w[q]);
}

// Expert totals (the words' popcounts, pc) and their exclusive scan into
// loffs[0..E] (LDS); work-group 0 also stores them to expert_offsets.  E <= 8.
// All threads call it.
__device__ __forceinline__ void mask_offsets(const uint32_t (&pc)[kOffWords], int E, int nwords, int32_t *ltot,
                                             int32_t *loffs, int32_t *__restrict__ expert_offsets)
{
    const int tid = threadIdx.x;
    if (tid < E)
        ltot[tid] = 0;
    int cnt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        cnt[e] = 0;
#pragma unroll
    for (int q = 0; q < kOffWords; ++q) {
        const int ex = (tid + q * kBlock) / nwords;   // >= E past the end, where the word is 0
#pragma unroll
        for (int e = 0; e < 8; ++e)
            cnt[e] += ex == e ? (int)pc[q] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e >= E)
            break;
        int v = cnt[e];
        for (int o = kWave / 2; o > 0; o >>= 1)
            v += __shfl_xor(v, o);
        if (lane_id() == 0)
            atomicAdd(&ltot[e], v);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            loffs[e] = run;
            run += ltot[e];
        }
        loffs[E] = run;
    }
    __syncthreads();
    if (blockIdx.x == 0 && tid <= E)
        expert_offsets[tid] = loffs[tid];
}

__device__ __forceinline__ void route_logits_load(const float *__restrict__ logits, int64_t T, int E,
                                                  float (&v)[kRoutePasses], uint32_t (&key)[kRoutePasses])
{
    const int gl = lane_id() % 8;
#pragma unroll
    for (int p = 0; p < kRoutePasses; ++p) {
        const int64_t tt = p * kMaskChunk + (int)threadIdx.x / 8;
        float vv[1];
        uint32_t kk[1];
        route_core::load_logits<1, false>(logits, tt, tt < T, E, gl, vv, kk);
        v[p] = vv[0];
        key[p] = kk[0];
    }
}

__device__ __forceinline__ void route_local_counts(const float (&v)[kRoutePasses], const uint32_t (&key)[kRoutePasses],
                                                   int64_t T, int E, int k, bool packed, int32_t *__restrict__ out_idx,
                                                   float *__restrict__ out_w, uint32_t *lmask, int32_t *lids,
                                                   int32_t *loffs, int32_t *wave_sums,
                                                   int32_t *__restrict__ expert_counts,
                                                   int32_t *__restrict__ expert_offsets)
{
    const int tid = threadIdx.x;
    const int gl = lane_id() % 8;
    for (int i = tid; i < E * kMaskStride; i += kBlock)
        lmask[i] = 0u;
    __syncthreads();
    const bool store = blockIdx.x == 0;
#pragma unroll
    for (int p = 0; p < kRoutePasses; ++p) {
        if (p * kMaskChunk >= T)   // uniform: T is the same for the whole work-group
            break;
        const int64_t tt = p * kMaskChunk + tid / 8;
        const bool active = tt < T;
        const float vv[1] = {v[p]};
        uint32_t kk[1] = {key[p]};
        const int e = route_core::select_and_store<8, 1>(vv, kk, active, tt, E, k, store ? out_idx : nullptr,
                                                         store ? out_w : nullptr);
        if (active && gl < k) {
            lids[tt * k + gl] = e;
            atomicOr(&lmask[e * kMaskStride + ((int)tt >> 5)], 1u << ((int)tt & 31));
        }
    }
    __syncthreads();
    local_totals(E, kMaskWords, kMaskStride, packed, lmask, loffs, wave_sums, expert_counts, expert_offsets);
}

// The expert id (and for 256-token chunks the in-chunk rank) of pair
// (t, lane / lanes_per_pair); -1 for lanes that own no pair.
struct PairIds {
    int e, r;
};

__device__ __forceinline__ PairIds load_pair_ids(const int32_t *__restrict__ topk_idx,
                                                 const int32_t *__restrict__ local_rank, bool active, int64_t t, int k,
                                                 int lanes_per_pair)
{
    const int j = lane_id() / lanes_per_pair;
    const bool own = active && j < k;
    const int64_t q = (active ? t : 0) * k + (j < k ? j : k - 1);
    const int e = topk_idx[q];
    const int r = local_rank ? local_rank[q] : -1;
    return {own ? e : -1, own ? r : -1};
}

// Slot of pair (t, j) for the lanes that own it, -1 elsewhere.  L =
// lanes_per_pair lanes serve pair j = lane / L: they load the expert id and
// in-chunk rank (or take them from `pre` when PRE, the single-chunk
// kernels), and sum the expert's counts over all earlier 256-token chunks
// (the exclusive prefix, read from the L2-resident chunk histograms in
// groups of eight per lane), then a butterfly within the L lanes.  Fixed slots (offs == NULL): slot = e*C + prefix +
// rank, or -1 when that is >= C.  Packed (offs != NULL): slot = offs[e] +
// prefix + rank.  -1 for an id out of range.  The value is valid in lane
// j*L.
//
// With masks != NULL the counts come from the router's 32-token membership
// words instead (bit b of masks[e][c] = token 32c + b chose e): the prefix
// sums the popcounts of the expert's earlier words and the rank is the
// popcount of its own word below the token's bit.
//
// SCANNED: chunk_counts already holds each expert's exclusive prefix over
// chunks, so the prefix is one load.
//
// With lmask != NULL (a single chunk, masks rebuilt in LDS) the rank comes
// from the LDS words and there is no earlier chunk.  With loffs != NULL the
// packed offsets are read from LDS instead of offs.
template <bool PRE, bool SCANNED = false>
__device__ __forceinline__ int wave_slot(PairIds pre, const int32_t *__restrict__ topk_idx,
                                         const int32_t *__restrict__ local_rank,
                                         const int32_t *__restrict__ chunk_counts, const uint32_t *__restrict__ masks,
                                         const int32_t *__restrict__ offs, const uint32_t *lmask, const int32_t *loffs,
                                         int64_t t, int E, int k, int C, int nchunks, int lanes_per_pair, int ns)
{
    const int lane = lane_id();
    const int j = lane / lanes_per_pair;
    const int sub = lane - j * lanes_per_pair;
    const int c = (int)(masks ? t / kMaskChunk : t / kChunk);
    int e = -1, r = -1, sum = 0, base = 0;
    if (j < k) {
        e = PRE ? pre.e : topk_idx[t * k + j];
        if ((unsigned)e < (unsigned)E) {
            if (offs)
                base = loffs ? loffs[e] : offs[e];
            if (lmask) {   // the earlier words' popcounts, spread over the pair's lanes
                const int word = (int)t >> 5;
                const uint32_t *row = lmask + e * ns;
                r = __popc(row[word] & ((1u << ((int)t & 31)) - 1u));
                for (int w = sub; w < word; w += lanes_per_pair)
                    sum += __popc(row[w]);
            } else if (masks) {
                const uint32_t *row = masks + (int64_t)e * nchunks;
                r = __popc(row[c] & ((1u << (int)(t % kMaskChunk)) - 1u));
                for (int b0 = sub; b0 < c; b0 += 8 * lanes_per_pair) {
                    uint32_t part[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int cc = b0 + u * lanes_per_pair;
                        part[u] = cc < c ? row[cc] : 0u;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        sum += __popc(part[u]);
                }
            } else {
                r = PRE ? pre.r : local_rank[t * k + j];
                const int32_t *row = chunk_counts + (int64_t)e * nchunks;
                if (SCANNED) {
                    if (sub == 0)
                        sum = row[c];   // already the prefix over chunks 0 .. c-1
                } else {
                    for (int b0 = sub; b0 < c; b0 += 8 * lanes_per_pair) {
                        int part[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int cc = b0 + u * lanes_per_pair;
                            part[u] = cc < c ? row[cc] : 0;
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u)
                            sum += part[u];
                    }
                }
            }
        }
    }
    sum = group_sum(sum, lanes_per_pair);
    int slot = -1;
    if (j < k && (unsigned)e < (unsigned)E && r >= 0) {
        if (offs)
            slot = base + sum + r;
        else if ((int64_t)sum + r < C)
            slot = (int)((int64_t)e * C + sum + r);
    }
    return slot;
}

// Segment 0 of each token records token_slot and recv_src.
__device__ __forceinline__ void record_slot(int slot, int64_t t, int k, int lanes_per_pair,
                                            int32_t *__restrict__ token_slot, int32_t *__restrict__ recv_src)
{
    const int lane = lane_id();
    const int j = lane / lanes_per_pair;
    if (j < k && lane == j * lanes_per_pair) {
        token_slot[t * k + j] = slot;
        if (slot >= 0)
            recv_src[slot] = (int32_t)t;
    }
}

// The true per-expert totals, spread over the first waves of the grid
// (from the chunk histograms, or the popcounts of the router's masks).
__device__ __forceinline__ void wave_totals(int64_t task, int64_t ntasks, const int32_t *__restrict__ chunk_counts,
                                            const uint32_t *__restrict__ masks, int E, int nchunks,
                                            int32_t *__restrict__ expert_counts)
{
    const int lane = lane_id();
    for (int64_t e = task; e < E; e += ntasks) {
        int sum = 0;
        for (int cc = lane; cc < nchunks; cc += kWave)
            sum += masks ? __popc(masks[e * nchunks + cc]) : chunk_counts[e * nchunks + cc];
        for (int o = kWave / 2; o > 0; o >>= 1)
            sum += __shfl_xor(sum, o);
        if (lane == 0)
            expert_counts[e] = sum;
    }
}

constexpr int kMaxV = 16;  // most 16-byte vectors per lane in flight (bf16 rows)

// bf16 rows: one wave per (token, row segment).  The lane's vectors
// seg*VPL*64 + i*64 + lane (i < VPL) are all requested first, then the
// slots are worked out, then every vector is stored to each of the k slots.
// LOCAL (a single 256-token chunk): the work-group first rebuilds the
// chunk's masks in LDS (two barriers) from ids requested before the rows.
// Otherwise there is no work-group barrier and the waves' latency chains
// overlap freely.
template <int VPL, int MODE>
__global__ __launch_bounds__(kBlock) void dispatch_pack_bf16_kernel(
    const u32x4 *__restrict__ x, int64_t T, int nvec, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ local_rank, const int32_t *__restrict__ chunk_counts,
    const uint32_t *__restrict__ masks, int32_t *offs, int E, int k, int C, int nchunks, int lanes_per_pair,
    int segs,
    int32_t *__restrict__ token_slot, int32_t *__restrict__ recv_src, int32_t *__restrict__ expert_counts,
    u32x4 *__restrict__ recv_x, const float *__restrict__ logits, int32_t *__restrict__ route_idx,
    float *__restrict__ route_w)
{
    constexpr bool LIDS = local_ids_mode<MODE>();
    constexpr bool LOCAL = LIDS || MODE == kPackLocalRoute;
    extern __shared__ uint32_t lds_words[];  // local counting only: masks, packed offsets, routed ids
    __shared__ int32_t wave_sums[kWavesPerBlock];
    uint32_t *lmask = LOCAL ? lds_words : nullptr;
    const int nw = local_words(T);   // LDS membership words per expert (local modes)
    const int ns = local_stride(nw); // and the row stride of the masks
    int32_t *loffs = LOCAL && offs ? (int32_t *)(lds_words + E * ns)
                     : MODE == kPackMaskOffsets ? (int32_t *)(lds_words + E) : nullptr;
    const int lane = lane_id();
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    const bool active = t < T;
    const u32x4 *src = x + (active ? t : 0) * nvec;
    const int v0 = seg * VPL * kWave + lane;
    // One chunk: the ids are requested first and the row loads carry no
    // branch, so the LDS counting waits for the ids but not for the rows.
    // Otherwise wave_slot loads the ids after the rows are requested (moving
    // them ahead was measured slower there).
    PairIds ids = {-1, -1};
    int lids[local_ids_count<MODE>()];
    float rv[kRoutePasses];
    uint32_t rkey[kRoutePasses];
    if (LIDS) {
        ids = load_pair_ids(topk_idx, local_rank, active, t, k, lanes_per_pair);
        local_ids_load(topk_idx, (int)T * k, lids);
    }
    if (MODE == kPackLocalRoute)
        route_logits_load(logits, T, E, rv, rkey);
    uint32_t mw[kOffWords];
    if (MODE == kPackMaskOffsets)
        mask_words_load(masks, E * nchunks, mw);
    u32x4 buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v0 + i * kWave;
        if (LOCAL || MODE == kPackMaskOffsets)   // lanes past the row end load its last vector, store nothing
            buf[i] = src[v < nvec ? v : nvec - 1];
        else
            buf[i] = active && v < nvec ? src[v] : (u32x4){0, 0, 0, 0};
    }
    if (MODE == kPackMaskOffsets)
        mask_words_count(mw);
    // (local counting overlaps the row loads; every thread takes part)
    int32_t *lroute = (int32_t *)(lds_words + E * ns + E + 1);   // routed ids [T][k]
    if (LIDS)
        local_chunk_counts(lids, E, k, nw, ns, offs != nullptr, lds_words, (int32_t *)(lds_words + E * ns),
                           wave_sums, expert_counts, offs);
    if (MODE == kPackLocalRoute) {
        route_local_counts(rv, rkey, T, E, k, offs != nullptr, route_idx, route_w, lds_words, lroute,
                           (int32_t *)(lds_words + E * ns), wave_sums, expert_counts, offs);
        const int j = lane / lanes_per_pair;
        ids.e = active && j < k ? lroute[t * k + j] : -1;
    }
    if (MODE == kPackMaskOffsets)
        mask_offsets(mw, E, nchunks, (int32_t *)lds_words, loffs, offs);
    if (!active)
        return;

    const int slot = wave_slot<LOCAL, MODE == kPackScanned>(ids, topk_idx, local_rank, chunk_counts, masks, offs,
                                                             lmask, loffs, t, E, k, C, nchunks, lanes_per_pair,
                                                             ns);
    if (seg == 0)
        record_slot(slot, t, k, lanes_per_pair, token_slot, recv_src);
    if (task < E && expert_counts && !LOCAL && MODE != kPackScanned)
        wave_totals(task, T * segs, chunk_counts, masks, E, nchunks, expert_counts);

#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        const int s = lane_value(slot, j * lanes_per_pair);
        if (s < 0)
            continue;
        u32x4 *dst = recv_x + (int64_t)s * nvec;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (v0 + i * kWave < nvec)
                store_stream(dst + v0 + i * kWave, buf[i]);
    }
}

constexpr int kMaxG = 8;   // most 16-element groups per lane in flight (fp8 rows)

// fp8 rows: one wave per (token, row segment); a lane owns groups of 16
// consecutive elements (two 16-byte loads, one 16-byte code store), groups
// seg*VPL*64 + i*64 + lane.  The 8 consecutive lanes holding one
// 128-element block find its amax with three DPP steps; the scale is
// amax/448 (IEEE division; 1 for an all-zero block) and each code is the
// E4M3 encoding (round to nearest even, saturating) of x / scale, with the
// quotient bit-identical to an IEEE division (divide_all).  The load order
// and LOCAL are as in the bf16 kernel.
template <int VPL, int MODE>
__global__ __launch_bounds__(kBlock) void dispatch_pack_fp8_kernel(
    const u32x4 *__restrict__ x, int64_t T, int ngrp, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ local_rank, const int32_t *__restrict__ chunk_counts,
    const uint32_t *__restrict__ masks, int32_t *offs, int E, int k, int C, int nchunks, int lanes_per_pair,
    int segs,
    int32_t *__restrict__ token_slot, int32_t *__restrict__ recv_src, int32_t *__restrict__ expert_counts,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_scales, const float *__restrict__ logits,
    int32_t *__restrict__ route_idx, float *__restrict__ route_w)
{
    constexpr bool LIDS = local_ids_mode<MODE>();
    constexpr bool LOCAL = LIDS || MODE == kPackLocalRoute;
    // the wave's block scales, staged so each slot's scale segment is
    // written by one contiguous store instruction
    __shared__ float s_scale[kWavesPerBlock][VPL * 8];
    float *my_scale = s_scale[threadIdx.x / kWave];
    extern __shared__ uint32_t lds_words[];  // local counting only: masks, then packed offsets
    __shared__ int32_t wave_sums[kWavesPerBlock];
    uint32_t *lmask = LOCAL ? lds_words : nullptr;
    const int nw = local_words(T);   // LDS membership words per expert (local modes)
    const int ns = local_stride(nw); // and the row stride of the masks
    int32_t *loffs = LOCAL && offs ? (int32_t *)(lds_words + E * ns)
                     : MODE == kPackMaskOffsets ? (int32_t *)(lds_words + E) : nullptr;
    const int lane = lane_id();
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int64_t t = task / segs;
    const int seg = (int)(task - t * segs);
    const bool active = t < T;
    const u32x4 *src = x + (active ? t : 0) * (int64_t)ngrp * 2;
    const int nblk = ngrp / 8;
    const int g0 = seg * VPL * kWave + lane;
    PairIds ids = {-1, -1};   // the same load order as the bf16 kernel
    int lids[local_ids_count<MODE>()];
    float rv[kRoutePasses];
    uint32_t rkey[kRoutePasses];
    if (LIDS) {
        ids = load_pair_ids(topk_idx, local_rank, active, t, k, lanes_per_pair);
        local_ids_load(topk_idx, (int)T * k, lids);
    }
    if (MODE == kPackLocalRoute)
        route_logits_load(logits, T, E, rv, rkey);
    uint32_t mw[kOffWords];
    if (MODE == kPackMaskOffsets)
        mask_words_load(masks, E * nchunks, mw);
    u32x4 lo[VPL], hi[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int g = g0 + i * kWave;
        if (LOCAL || MODE == kPackMaskOffsets) {   // lanes past the row end load its last group, store nothing
            const int gc = g < ngrp ? g : ngrp - 1;
            lo[i] = src[2 * gc];
            hi[i] = src[2 * gc + 1];
        } else {
            lo[i] = hi[i] = (u32x4){0, 0, 0, 0};
            if (active && g < ngrp) {
                lo[i] = src[2 * g];
                hi[i] = src[2 * g + 1];
            }
        }
    }
    if (MODE == kPackMaskOffsets)
        mask_words_count(mw);
    // (local counting overlaps the row loads; every thread takes part)
    int32_t *lroute = (int32_t *)(lds_words + E * ns + E + 1);   // routed ids [T][k]
    if (LIDS)
        local_chunk_counts(lids, E, k, nw, ns, offs != nullptr, lds_words, (int32_t *)(lds_words + E * ns),
                           wave_sums, expert_counts, offs);
    if (MODE == kPackLocalRoute) {
        route_local_counts(rv, rkey, T, E, k, offs != nullptr, route_idx, route_w, lds_words, lroute,
                           (int32_t *)(lds_words + E * ns), wave_sums, expert_counts, offs);
        const int j = lane / lanes_per_pair;
        ids.e = active && j < k ? lroute[t * k + j] : -1;
    }
    if (MODE == kPackMaskOffsets)
        mask_offsets(mw, E, nchunks, (int32_t *)lds_words, loffs, offs);
    if (!active)
        return;

    const int slot = wave_slot<LOCAL, MODE == kPackScanned>(ids, topk_idx, local_rank, chunk_counts, masks, offs,
                                                             lmask, loffs, t, E, k, C, nchunks, lanes_per_pair,
                                                             ns);
    if (seg == 0)
        record_slot(slot, t, k, lanes_per_pair, token_slot, recv_src);
    if (task < E && expert_counts && !LOCAL && MODE != kPackScanned)
        wave_totals(task, T * segs, chunk_counts, masks, E, nchunks, expert_counts);

#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int g = g0 + i * kWave;   // the 8 lanes of a scale block share validity (ngrp % 8 == 0)
        float f[16];
        const uint32_t w[8] = {lo[i][0], lo[i][1], lo[i][2], lo[i][3], hi[i][0], hi[i][1], hi[i][2], hi[i][3]};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            f[2 * q] = bf16_lo(w[q]);
            f[2 * q + 1] = bf16_hi(w[q]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            amax = fmaxf(amax, fabsf(f[q]));
        amax = group_max<8>(amax);
        if (g >= ngrp)
            continue;
        const float sc = block_scale(amax);
        const u32x4 codes = quantize16(f, sc);
        if ((lane & 7) == 0)
            my_scale[i * 8 + lane / 8] = sc;
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            const int s = lane_value(slot, j * lanes_per_pair);
            if (s < 0)
                continue;
            store_stream(recv_x + (int64_t)s * ngrp + g, codes);
        }
    }
    // scales of this segment's blocks blk0 .. blk0+nb-1, one lane each
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int blk0 = seg * VPL * 8;
    const int nb = min(VPL * 8, nblk - blk0);
    if (lane < nb) {
        const float v = my_scale[lane];
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            const int s = lane_value(slot, j * lanes_per_pair);
            if (s >= 0)
                store_stream(recv_scales + (int64_t)s * nblk + blk0 + lane, v);
        }
    }
}

// Lanes per (t, j) pair in the slot computation: 64 / next_pow2(k).
int pair_lanes(int k)
{
    int p = 1;
    while (p < k)
        p <<= 1;
    return kWave / p;
}

// Units (vectors or groups) per lane and row segments per token.  A lane
// aims at about eight row stores in flight: `target` units per lane (8 / k
// for bf16 rows, whose unit is one 16-byte store per copy; 2 for fp8, whose
// unit already reads 32 bytes).  Fewer, longer waves also repeat the slot
// lookup fewer times per token.  Measured with rotated buffers: at 4096
// tokens of width 4096, top-2, four vectors per lane beat two by 2.4 us;
// at 16384 tokens of width 7168, top-8, one beats two; fp8 rows are fastest
// at two.  The count halves while the grid would hold fewer than 2048 waves,
// so small batches still spread over the chip.
void choose_split(int64_t T, int nunits, int max_per_lane, int target, int *vpl, int *segs)
{
    int v = 1;
    while (v * 2 <= target && v * 2 <= max_per_lane)
        v *= 2;
    while (v > 1 && T * ((nunits + v * kWave - 1) / (v * kWave)) < 2048)
        v /= 2;
    while (v < max_per_lane && T * ((nunits + v * kWave - 1) / (v * kWave)) * kWave > kMaxGridItems)
        v *= 2;
    *vpl = v;
    *segs = (nunits + v * kWave - 1) / (v * kWave);
}

// The pack grid for rows of width H: vectors (bf16) or 16-element groups
// (fp8) per lane, and row segments per token.  False when the grid would
// exceed the launch limit.
bool pack_split(int64_t T, int H, int k, int dtype, int *vpl, int *segs)
{
    if (dtype == 0)
        choose_split(T, H / 8, kMaxV, k >= 8 ? 1 : 8 / k, vpl, segs);
    else
        choose_split(T, H / 16, kMaxG, 2, vpl, segs);
    return grid_fits((T * *segs + kWavesPerBlock - 1) / kWavesPerBlock, kBlock);
}

// The pack launch shared by every path: `masks` (router membership words of
// 32-token chunks) or chunk_counts + local_rank (256-token chunks) give the
// counts; offs selects the packed layout.
hipError_t launch_pack(const uint16_t *x, int64_t T, int H, const int32_t *topk_idx, const int32_t *local_rank,
                       const int32_t *chunk_counts, const uint32_t *masks, int32_t *offs, int E, int k, int C,
                       int nchunks, int dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                       int32_t *expert_counts, int32_t *token_slot, hipStream_t s, int mode = kPackChunks,
                       const float *logits = nullptr, int32_t *route_idx = nullptr, float *route_w = nullptr)
{
    // single chunk: masks [E][9] (or [E][nw | 1]) and offsets [E+1] in LDS (+ routed ids [T][k]);
    // totals from membership words: totals [E] and offsets [E+1]
    const size_t lds = mode == kPackChunks || mode == kPackScanned ? 0
                     : mode == kPackMaskOffsets ? (size_t)(2 * E + 1) * 4
                     : (size_t)(E * local_stride(local_words(T)) + E + 1 + (mode == kPackLocalRoute ? T * k : 0)) * 4;
    const int lpp = pair_lanes(k);
    int vpl, segs;
    if (!pack_split(T, H, k, dtype, &vpl, &segs))
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((T * segs + kWavesPerBlock - 1) / kWavesPerBlock));
    if (dtype == 0) {
        const int nvec = H / 8;
#define MOE_PACK_BF16_L(V, M)                                                                                      \
    hipLaunchKernelGGL((dispatch_pack_bf16_kernel<V, M>), grid, dim3(kBlock), lds, s, (const u32x4 *)x, T, nvec,      \
                       topk_idx, local_rank, chunk_counts, masks, offs, E, k, C, nchunks, lpp, segs, token_slot,           \
                       recv_src, expert_counts, (u32x4 *)recv_x, logits, route_idx, route_w)
#define MOE_PACK_BF16(V)                                                                                         \
    do {                                                                                                         \
        if (mode == kPackLocalRoute)                                                                             \
            MOE_PACK_BF16_L(V, kPackLocalRoute);                                                                 \
        else if (mode == kPackLocalIds)                                                                          \
            MOE_PACK_BF16_L(V, kPackLocalIds);                                                                   \
        else if (mode == kPackLocalIdsWide)                                                                      \
            MOE_PACK_BF16_L(V, kPackLocalIdsWide);                                                               \
        else if (mode == kPackMaskOffsets)                                                                       \
            MOE_PACK_BF16_L(V, kPackMaskOffsets);                                                                \
        else if (mode == kPackScanned)                                                                           \
            MOE_PACK_BF16_L(V, kPackScanned);                                                                    \
        else                                                                                                     \
            MOE_PACK_BF16_L(V, kPackChunks);                                                                     \
    } while (0)
        switch (vpl) {
        case 1: MOE_PACK_BF16(1); break;
        case 2: MOE_PACK_BF16(2); break;
        case 4: MOE_PACK_BF16(4); break;
        case 8: MOE_PACK_BF16(8); break;
        default: MOE_PACK_BF16(16); break;
        }
#undef MOE_PACK_BF16
#undef MOE_PACK_BF16_L
    } else {
        const int ngrp = H / 16;
#define MOE_PACK_FP8_L(V, M)                                                                                       \
    hipLaunchKernelGGL((dispatch_pack_fp8_kernel<V, M>), grid, dim3(kBlock), lds, s, (const u32x4 *)x, T, ngrp,       \
                       topk_idx, local_rank, chunk_counts, masks, offs, E, k, C, nchunks, lpp, segs, token_slot,           \
                       recv_src, expert_counts, (u32x4 *)recv_x, recv_scales, logits, route_idx, route_w)
#define MOE_PACK_FP8(V)                                                                                          \
    do {                                                                                                         \
        if (mode == kPackLocalRoute)                                                                             \
            MOE_PACK_FP8_L(V, kPackLocalRoute);                                                                  \
        else if (mode == kPackLocalIds)                                                                          \
            MOE_PACK_FP8_L(V, kPackLocalIds);                                                                    \
        else if (mode == kPackLocalIdsWide)                                                                      \
            MOE_PACK_FP8_L(V, kPackLocalIdsWide);                                                                \
        else if (mode == kPackMaskOffsets)                                                                       \
            MOE_PACK_FP8_L(V, kPackMaskOffsets);                                                                 \
        else if (mode == kPackScanned)                                                                           \
            MOE_PACK_FP8_L(V, kPackScanned);                                                                     \
        else                                                                                                     \
            MOE_PACK_FP8_L(V, kPackChunks);                                                                      \
    } while (0)
        switch (vpl) {
        case 1: MOE_PACK_FP8(1); break;
        case 2: MOE_PACK_FP8(2); break;
        case 4: MOE_PACK_FP8(4); break;
        default: MOE_PACK_FP8(8); break;
        }
#undef MOE_PACK_FP8
#undef MOE_PACK_FP8_L
    }
    return hipGetLastError();
}

}  // namespace

bool dispatch_grid_fits(int64_t T, int H, int k, int dtype)
{
    int vpl, segs;
    return pack_split(T, H, k, dtype, &vpl, &segs);
}

size_t dispatch_workspace_bytes(int64_t T, int E, int k)
{
    const int64_t nchunks = (T + kChunk - 1) / kChunk;
    const int64_t a = ((int64_t)E * nchunks * 4 + 255) / 256 * 256;
    const int64_t b = (T * k * 4 + 255) / 256 * 256;
    return (size_t)(a + b);
}

hipError_t launch_dispatch(const uint16_t *x, int64_t T, int H, const int32_t *topk_idx, int E, int k, int C,
                           int dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                           int32_t *expert_counts, int32_t *expert_offsets, int32_t *token_slot, void *workspace,
                           hipStream_t s)
{
    if (T == 0) {
        int32_t *zero = expert_offsets ? expert_offsets : expert_counts;
        const int n = expert_offsets ? E + 1 : E;
        hipLaunchKernelGGL(dispatch_zero_counts_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, zero, n);
        return hipGetLastError();
    }
    if (!dispatch_grid_fits(T, H, k, dtype))   // before anything is enqueued
        return hipErrorInvalidConfiguration;
    const int nchunks = (int)((T + kChunk - 1) / kChunk);
    // pack counts the whole batch itself, no count launch
    if (local_count(T, E, k))
        return launch_pack(x, T, H, topk_idx, nullptr, nullptr, nullptr, expert_offsets, E, k, C, 1, dtype, recv_x,
                           recv_scales, recv_src, expert_counts, token_slot, s,
                           local_ids_wide(T, k) ? kPackLocalIdsWide : kPackLocalIds);
    int32_t *chunk_counts = (int32_t *)workspace;
    int32_t *local_rank =
        (int32_t *)((char *)workspace + ((int64_t)E * nchunks * 4 + 255) / 256 * 256);

    // packed layout: one more work-group totals the chunks and scans
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kBlock), (size_t)E * kCountStride * 4, s, topk_idx,
                       T, E, k, nchunks, chunk_counts, local_rank);
    if (expert_offsets)
        hipLaunchKernelGGL(dispatch_offsets_kernel<false>, dim3(1), dim3(kScanBlock), 0, s, chunk_counts, E,
                           nchunks, expert_offsets);
    int32_t *offs = expert_offsets;
    if (nchunks > kScanChunks) {   // prefixes scanned once; the scan also writes the totals
        hipLaunchKernelGGL(dispatch_chunk_scan_kernel, dim3(E), dim3(kBlock), 0, s, chunk_counts, nchunks,
                           expert_counts);
        return launch_pack(x, T, H, topk_idx, local_rank, chunk_counts, nullptr, offs, E, k, C, nchunks, dtype,
                           recv_x, recv_scales, recv_src, nullptr, token_slot, s, kPackScanned);
    }

    return launch_pack(x, T, H, topk_idx, local_rank, chunk_counts, nullptr, offs, E, k, C, nchunks, dtype, recv_x,
                       recv_scales, recv_src, expert_counts, token_slot, s);
}

hipError_t launch_route_dispatch(const float *logits, int64_t T, int E, int k, const uint16_t *x, int H, int C,
                                 int dtype, int32_t *topk_idx, float *topk_w, void *recv_x, float *recv_scales,
                                 int32_t *recv_src, int32_t *expert_counts, int32_t *expert_offsets,
                                 int32_t *token_slot, void *workspace, hipStream_t s)
{
    if (T == 0) {
        int32_t *zero = expert_offsets ? expert_offsets : expert_counts;
        const int n = expert_offsets ? E + 1 : E;
        hipLaunchKernelGGL(dispatch_zero_counts_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, zero, n);
        return hipGetLastError();
    }
    if (!dispatch_grid_fits(T, H, k, dtype))
        return hipErrorInvalidConfiguration;
    // E <= 8 and one 256-token chunk: one launch, every pack work-group
    // routes the whole batch itself (route_local_counts).
    // E <= 8 beyond that: the router writes 32-token membership words and
    // pack derives the slots from them (two launches; for the packed layout
    // every pack work-group also totals the words into the offsets, or for
    // more than 2048 words one added work-group does it first).
    // Otherwise, or when the prefix over those words would exceed
    // mask_prefix_loads per lane: route, count (+ offsets), pack -- or for a
    // batch pack can count, route and a pack that counts in LDS.
    if (E <= 8 && T <= kChunk)
        return launch_pack(x, T, H, nullptr, nullptr, nullptr, nullptr, expert_offsets, E, k, C, 1, dtype, recv_x,
                           recv_scales, recv_src, expert_offsets ? nullptr : expert_counts, token_slot, s,
                           kPackLocalRoute, logits, topk_idx, topk_w);
    const int64_t nmask = (T + kMaskChunk - 1) / kMaskChunk;
    const int lpp = pair_lanes(k);
    if (E <= 8 && nmask <= mask_prefix_loads(E, k) * (int64_t)lpp &&
        (size_t)E * nmask * 4 <= dispatch_workspace_bytes(T, E, k)) {
        uint32_t *masks = (uint32_t *)workspace;
        hipError_t e = launch_route_topk_masks(logits, T, E, k, topk_idx, topk_w, masks, s);
        if (e != hipSuccess)
            return e;
        // packed: each pack work-group totals the words itself while they fit
        // kOffWords per thread, else one work-group does it first
        const bool own_offsets = expert_offsets && E * nmask <= (int64_t)kOffWords * kBlock;
        if (expert_offsets && !own_offsets)
            hipLaunchKernelGGL(dispatch_offsets_kernel<true>, dim3(1), dim3(kScanBlock), 0, s,
                               (const int32_t *)masks, E, (int)nmask, expert_offsets);
        return launch_pack(x, T, H, topk_idx, nullptr, nullptr, masks, expert_offsets, E, k, C, (int)nmask, dtype,
                           recv_x, recv_scales, recv_src, expert_offsets ? nullptr : expert_counts, token_slot, s,
                           own_offsets ? kPackMaskOffsets : kPackChunks);
    }
    // E > 8, fixed slots, a batch past the in-pack count with few enough
    // membership words: the router writes the words a 16-token half per
    // work-group and pack derives the slots from them, as for E <= 8 (two
    // launches instead of three).
    if (E > 8 && !expert_offsets && !local_count(T, E, k) && nmask <= mask_prefix_loads(E, k) * (int64_t)lpp &&
        (size_t)E * nmask * 4 <= dispatch_workspace_bytes(T, E, k)) {
        uint32_t *masks = (uint32_t *)workspace;
        hipError_t e = launch_route_topk_half_masks(logits, T, E, k, topk_idx, topk_w, masks, s);
        if (e != hipSuccess)
            return e;
        return launch_pack(x, T, H, topk_idx, nullptr, nullptr, masks, nullptr, E, k, C, (int)nmask, dtype, recv_x,
                           recv_scales, recv_src, expert_counts, token_slot, s, kPackChunks);
    }
    hipError_t e = launch_route_topk(logits, T, E, k, topk_idx, topk_w, s);
    if (e != hipSuccess)
        return e;
    return launch_dispatch(x, T, H, topk_idx, E, k, C, dtype, recv_x, recv_scales, recv_src,
                           expert_offsets ? nullptr : expert_counts, expert_offsets, token_slot, workspace, s);
}

}  // namespace moe
