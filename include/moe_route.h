/*
 * moe_route.h -- C ABI of libmoe_route.so: Mixture-of-Experts token routing,
 * dispatch and combine on one AMD Instinct MI355X (gfx950).
 *
 * The three operations are those of an expert-parallel MoE layer, as the
 * following pages describe them:
 *   - Perplexity, "Efficient and portable mixture-of-experts communication"
 *     (pplx-kernels blog): Introduction (router, top-K, weighted sum),
 *     Portable kernels (fixed per-source buffers, reused across layers),
 *     Dispatch (pack tokens into contiguous per-expert buffers for the
 *     grouped GEMM, keep each token's source index), Combine (weighted sum
 *     of 16-bit expert outputs into a caller-allocated tensor).
 *   - "How GPUs Talk to Each Other During LLM Inference", section 7 (Expert
 *     Parallelism): dispatch groups tokens by expert; combine weights each
 *     expert output by the router's score and adds the k outputs.
 *   - AI-infra handbook, "NVSHMEM and DeepEP": "Why MoE's all-to-all is
 *     hard" (route, sort by destination, count, dispatch, combine),
 *     "High-throughput mode" (FP8 dispatch with one scale per 128 elements,
 *     BF16 combine), "Low-latency mode" (fixed slots per expert, no host
 *     synchronisation, graph-capturable; too few slots is an error).
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are HIP device pointers; the caller allocates
 *     and owns every buffer.  The library allocates nothing on these paths
 *     and keeps no state between calls, except moe_route_dispatch_noalloc's
 *     static per-GPU scratch array (documented there).
 *   - All work is enqueued on `stream` (NULL = the default stream) and the
 *     call returns without waiting: no device synchronisation and no
 *     device-to-host copy, so calls can be captured in a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued.  The
 *     return value is MOE_OK or a negative MOE_ERR_* code; on error nothing
 *     was enqueued.  MOE_ERR_HIP reports a failed kernel launch.
 *   - No output (workspace included) may overlap an input or another output
 *     over the bytes the call touches: MOE_ERR_INVALID.  Inputs may share
 *     memory.  The one exception is documented where it applies.
 *   - Arrays are dense and row-major.  bf16 values are passed as their
 *     16-bit patterns (uint16_t).  Buffers read or written in 16-byte
 *     vectors (x, recv_x, y, out) must be 16-byte aligned.
 *   - Results are deterministic: the same inputs give the same bits on
 *     every call, whatever the launch order of the work-groups.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID (-1)      /* null pointer, negative size, k outside [1, E], misalignment */
#define MOE_ERR_UNSUPPORTED (-2)  /* a size this library does not handle (limits below) */
#define MOE_ERR_WORKSPACE (-3)    /* workspace missing or smaller than moe_dispatch_workspace_bytes() */
#define MOE_ERR_HIP (-4)          /* a HIP launch failed */
#define MOE_ERR_SCRATCH (-5)      /* moe_route_dispatch_noalloc: the batch needs more workspace than
                                     MOE_NOALLOC_SCRATCH_BYTES */

/* Dispatch row formats. */
#define MOE_DTYPE_BF16 0          /* rows copied bit for bit, 2*H bytes */
#define MOE_DTYPE_FP8_E4M3 1      /* OCP E4M3 codes (H bytes) + one fp32 scale per 128 elements */

/* Limits. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_GROUPS 64         /* expert groups of moe_route_topk_grouped */
#define MOE_MAX_NORM_HIDDEN 16384 /* H of moe_combine_residual_rmsnorm */
#define MOE_MAX_TOKENS (1 << 24)  /* T above this is MOE_ERR_UNSUPPORTED */
#define MOE_NOALLOC_SCRATCH_BYTES (4 << 20)  /* static device scratch of moe_route_dispatch_noalloc */
/* Also MOE_ERR_UNSUPPORTED: a dispatch or combine shape whose single kernel
 * launch would need more than 2^32 - 1 work-items.  Each lane moves at least
 * 128 bytes of row data per copy, so only rows wider than 32768 elements at
 * MOE_MAX_TOKENS tokens come near it (about a terabyte of activations). */

/* Text for a status code (static storage, never NULL). */
MOE_API const char *moe_status_string(int status);

/*
 * moe_route_topk -- router top-k selection and weights.
 *
 * pplx blog, Introduction: the router produces a probability distribution
 * over experts, the top-K experts are chosen and their outputs are weighted
 * by that distribution.  "How GPUs Talk", section 7: each output is weighted
 * by the score the router gave its expert.
 *
 *   logits   (device, in)  float [T][E] router logits
 *   T        tokens, 0 <= T <= MOE_MAX_TOKENS (T = 0 enqueues nothing)
 *   E        experts, 1 <= E <= MOE_MAX_EXPERTS
 *   k        experts per token, 1 <= k <= min(E, MOE_MAX_TOPK)
 *   topk_idx (device, out) int32 [T][k]: the k experts with the largest
 *            logits in descending order; equal logits are ordered by
 *            ascending expert index, and -0.0 equals +0.0.  NaN logits are
 *            outside the domain.
 *   topk_w   (device, out) float [T][k]: softmax over all E logits of the
 *            token, evaluated at topk_idx (not renormalised over the k):
 *            exp(L[e] - max) / sum exp(L - max), computed in fp32.
 *   stream   HIP stream
 */
MOE_API int moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t k,
                           int32_t *topk_idx, float *topk_w, hipStream_t stream);

/*
 * moe_route_topk_grouped -- group-limited ("node-limited") router top-k.
 *
 * Handbook "NVSHMEM and DeepEP", "High-throughput mode": DeepSeek-V3 sends a
 * token to at most a few nodes; every node is scored by the sum of its two
 * best expert scores, only the best nodes are eligible, and the top experts
 * are then chosen among those nodes' experts.  Here a node is a group of
 * E / n_groups consecutive experts and an expert's score is its logit.
 *
 *   logits, T, E, k, topk_idx, topk_w, stream: as for moe_route_topk
 *   n_groups     groups, 1 <= n_groups <= MOE_MAX_GROUPS, E % n_groups == 0
 *                and E / n_groups >= 2
 *   topk_groups  eligible groups per token, 1 <= topk_groups <= n_groups,
 *                with topk_groups * (E / n_groups) >= k
 * Per token: a group's score is the fp32 sum of its two largest logits (a
 * repeated largest value counts twice); the topk_groups groups with the
 * largest scores are kept, equal scores ordered by ascending group index;
 * topk_idx holds the k largest logits among the kept groups' experts,
 * ordered as in moe_route_topk.  topk_w is unchanged by the limit: the full
 * softmax over all E logits at each chosen expert.  With topk_groups ==
 * n_groups the result equals moe_route_topk's.
 */
MOE_API int moe_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t k, int32_t n_groups,
                                   int32_t topk_groups, int32_t *topk_idx, float *topk_w, hipStream_t stream);

/*
 * Bytes of device workspace moe_dispatch needs for T tokens and E experts
 * (per-chunk expert histograms).  Host function; returns 0 for bad sizes.
 */
MOE_API size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_dispatch -- per-expert counts, fixed-slot assignment and row packing.
 *
 * Handbook "Why MoE's all-to-all is hard": after routing, tokens are sorted
 * by destination and counted per destination.  Handbook "Low-latency mode":
 * every expert owns a fixed number of slots (`capacity`) so a token's write
 * address is known without a host round trip.  pplx blog, Dispatch: tokens
 * are laid out contiguously per expert for the grouped GEMM, and each
 * token's source index is kept for combine.  Handbook "High-throughput
 * mode": FP8 dispatch uses one scale per 128 elements.
 *
 *   x             (device, in)  bf16 [T][H] token activations, 16 B aligned
 *   T             tokens, 0 <= T <= MOE_MAX_TOKENS (T = 0 still zeroes
 *                 expert_counts)
 *   H             hidden size; multiple of 8 (bf16) or of 128 (fp8)
 *   topk_idx      (device, in)  int32 [T][k]; each row holds k distinct
 *                 experts in [0, E).  An id outside [0, E) is dropped
 *                 (token_slot -1, not counted).  Repeated ids in one row
 *                 are outside the domain (memory-safe, result unspecified).
 *   E, k          as for moe_route_topk
 *   capacity      C, slots per expert, >= 1, with E*C <= INT32_MAX
 *   out_dtype     MOE_DTYPE_BF16 or MOE_DTYPE_FP8_E4M3
 *   recv_x        (device, out) [E][C][H] rows: bf16 (2H bytes each) or
 *                 E4M3 codes (H bytes each); 16 B aligned.  Slot r of expert
 *                 e holds the r-th token (in ascending token order) routed
 *                 to e.  Unfilled slots are not written.
 *   recv_scales   (device, out) float [E][C][H/128] for fp8 (amax/448 of
 *                 each 128-element block, 1.0 for an all-zero block; codes
 *                 are RNE(x / scale) saturated to +-448); NULL for bf16.
 *   recv_src      (device, out) int32 [E][C]: source token of each filled
 *                 slot; unfilled slots are not written.
 *   expert_counts (device, out) int32 [E]: true number of tokens routed to
 *                 each expert.  A value above C means overflow: the later
 *                 tokens of that expert were dropped.  The handbook treats
 *                 too few slots as a failure of the batch; here it is
 *                 reported on the device, so no host synchronisation is
 *                 needed, and the caller decides (fail, or split the batch).
 *   token_slot    (device, out) int32 [T][k]: e*C + r, the recv_x row of
 *                 (t, j), or -1 if dropped.  Combine reads it.
 *   workspace     (device, scratch) at least moe_dispatch_workspace_bytes()
 *                 bytes, 256 B aligned; contents need no initialisation and
 *                 are undefined afterwards.
 *   stream        HIP stream
 * Buffers must not overlap.
 */
MOE_API int moe_dispatch(const uint16_t *x, int64_t T, int32_t H, const int32_t *topk_idx,
                         int32_t E, int32_t k, int32_t capacity, int32_t out_dtype,
                         void *recv_x, float *recv_scales, int32_t *recv_src,
                         int32_t *expert_counts, int32_t *token_slot, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_dispatch -- moe_route_topk followed by moe_dispatch (fixed
 * slots) in one call.
 *
 * The same steps and citations as the two calls; every output (topk_idx,
 * topk_w, expert_counts, token_slot, recv_src, recv_x, recv_scales) is
 * identical to calling moe_route_topk and then moe_dispatch.  For E <= 8
 * the count step is folded into the router's kernel: a work-group that
 * routes 32 tokens also records which of them chose each expert, and the
 * pack derives counts, prefixes and ranks from those words, so the call is
 * two kernel launches instead of three.  With E <= 8 and at most 256 tokens
 * it is one launch: every pack work-group routes the whole batch itself with
 * the router's own code.  E <= 8 with more than 2048 * (64 / p) tokens
 * (p = k rounded up to a power of two; 1024 * (64 / p) for k > 4) uses
 * route, count and pack.  For
 * E > 8, batches the pack cannot count itself (above 256 or 1024 tokens) but
 * of at most 1024 * (64 / p) tokens take the same two-launch path, a
 * work-group of the router writing a 16-token half of each word, when the
 * words (E * ceil(T/32) * 4 bytes) fit the workspace; otherwise route, count
 * and pack, with a scan of the per-chunk counts before the pack past 65536
 * tokens.
 *
 *   logits, T, E, k, topk_idx, topk_w: as for moe_route_topk
 *   x, H, capacity, out_dtype, recv_x, recv_scales, recv_src, expert_counts,
 *   token_slot, workspace (moe_dispatch_workspace_bytes(T, E, k) bytes),
 *   workspace_bytes, stream: as for moe_dispatch
 * Buffers must not overlap.
 */
MOE_API int moe_route_dispatch(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x,
                               int32_t H, int32_t capacity, int32_t out_dtype, int32_t *topk_idx,
                               float *topk_w, void *recv_x, float *recv_scales, int32_t *recv_src,
                               int32_t *expert_counts, int32_t *token_slot, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_dispatch_noalloc -- moe_route_dispatch with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * Its per-chunk histograms, in-chunk ranks and router membership words live
 * in a static array of MOE_NOALLOC_SCRATCH_BYTES (4 MiB) in each GPU's
 * memory, which the library holds from the first call on that device until
 * the process ends.  The first call on a device (with it current) looks up
 * that array's device address; later calls reuse it.
 *
 *   Arguments, outputs and results: exactly those of moe_route_dispatch,
 *   minus workspace and workspace_bytes.
 *   Limit: moe_dispatch_workspace_bytes(T, E, k) <= MOE_NOALLOC_SCRATCH_BYTES
 *   (for example T * k up to about a million pairs), else MOE_ERR_SCRATCH
 *   and nothing is enqueued.  MOE_ERR_HIP if the address lookup fails.
 *   Every call on one GPU shares that GPU's array, and nothing in it needs
 *   to start at zero (each call writes what it reads).  Calls that overlap
 *   in time on one GPU (different streams, or different host threads
 *   without ordering) race on the array and give undefined results; calls
 *   on one stream, or ordered by events, do not.
 */
MOE_API int moe_route_dispatch_noalloc(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x,
                                       int32_t H, int32_t capacity, int32_t out_dtype, int32_t *topk_idx,
                                       float *topk_w, void *recv_x, float *recv_scales, int32_t *recv_src,
                                       int32_t *expert_counts, int32_t *token_slot, hipStream_t stream);

/*
 * moe_dispatch_packed -- per-expert counts, packed count-sized layout and
 * row packing.
 *
 * Handbook "NVSHMEM and DeepEP", "High-throughput mode": the number of
 * tokens bound for each destination is computed first, and the receive
 * buffer is sized by it rather than reserved for the worst case.  pplx
 * blog, Dispatch: each expert's tokens are contiguous for the grouped GEMM.
 * Here expert e's rows are expert_offsets[e] .. expert_offsets[e+1]-1, one
 * row per routed pair, with no slack between experts: the buffer needs T*k
 * rows at most, whatever the routing (no host round trip to size it).
 *
 *   x, T, H, topk_idx, E, k, out_dtype, workspace, workspace_bytes, stream:
 *                  as for moe_dispatch (the same workspace size)
 *   recv_x         (device, out) [T*k][H] rows: bf16 (2H bytes each) or E4M3
 *                  codes (H bytes each); 16 B aligned.  Row
 *                  expert_offsets[e] + r holds the r-th token (ascending
 *                  token order) routed to e.  Rows from expert_offsets[E]
 *                  on are not written.
 *   recv_scales    (device, out) float [T*k][H/128] for fp8, as for
 *                  moe_dispatch; NULL for bf16.
 *   recv_src       (device, out) int32 [T*k]: source token of each row
 *                  below expert_offsets[E].
 *   expert_offsets (device, out) int32 [E+1]: expert_offsets[e] = number of
 *                  pairs routed to experts below e; expert_offsets[E] = all
 *                  routed pairs (T*k when every id is valid).  Counts are
 *                  the differences.
 *   token_slot     (device, out) int32 [T][k]: the recv_x row of (t, j), or
 *                  -1 for an id outside [0, E) (dropped, not counted).
 * moe_combine reads a packed buffer as one expert with T*k slots (E = 1,
 * capacity = max(1, T*k)).  Buffers must not overlap.
 */
MOE_API int moe_dispatch_packed(const uint16_t *x, int64_t T, int32_t H, const int32_t *topk_idx,
                                int32_t E, int32_t k, int32_t out_dtype, void *recv_x, float *recv_scales,
                                int32_t *recv_src, int32_t *expert_offsets, int32_t *token_slot,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_dispatch_packed -- moe_route_topk followed by
 * moe_dispatch_packed in one call.
 *
 * The same steps and citations as the two calls; every output (topk_idx,
 * topk_w, expert_offsets, token_slot, recv_src, recv_x, recv_scales) is
 * identical to calling moe_route_topk and then moe_dispatch_packed.  For
 * E <= 8 and more than 256 tokens the count step is folded into the
 * router's kernel as in moe_route_dispatch, and the pack kernel's
 * work-groups total the router's membership words into the offsets
 * themselves: two kernel launches instead of four (three when there are more
 * than 2048 such words, E * ceil(T/32), and one work-group totals them
 * first).  With E <= 8 and at most 256 tokens it is one launch, as for
 * moe_route_dispatch.
 *
 *   logits, T, E, k, topk_idx, topk_w: as for moe_route_topk
 *   x, H, out_dtype, recv_x, recv_scales, recv_src, expert_offsets,
 *   token_slot, workspace (moe_dispatch_workspace_bytes(T, E, k) bytes),
 *   workspace_bytes, stream: as for moe_dispatch_packed
 * Buffers must not overlap.
 */
MOE_API int moe_route_dispatch_packed(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x,
                                      int32_t H, int32_t out_dtype, int32_t *topk_idx, float *topk_w,
                                      void *recv_x, float *recv_scales, int32_t *recv_src,
                                      int32_t *expert_offsets, int32_t *token_slot, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * moe_combine -- gather each token's k expert outputs and return their
 * router-weighted sum in the original token order.
 *
 * pplx blog, Combine: the routing table gives, per expert, which buffer to
 * read and which weight to apply; the weighted sum of the 16-bit expert
 * outputs is written to a caller-allocated tensor.  "How GPUs Talk",
 * section 7: the k weighted outputs are added at the token's origin.
 *
 *   y          (device, in)  bf16 [E][C][H] expert outputs, same row layout
 *              as moe_dispatch's recv_x; 16 B aligned.  All E*C rows must
 *              be readable memory (unfilled rows may hold anything): the
 *              kernel may load row 0 in place of a skipped pair
 *   E, capacity, H   as for moe_dispatch (H multiple of 8)
 *   token_slot (device, in)  int32 [T][k] from moe_dispatch; entries < 0
 *              or >= E*C are skipped (left out of the sum)
 *   topk_w     (device, in)  float [T][k] router weights
 *   T, k       tokens (0..MOE_MAX_TOKENS) and experts per token
 *              (1..MOE_MAX_TOPK)
 *   out        (device, out) bf16 [T][H]; out[t][h] = bf16 RNE of
 *              acc, acc = +0 then acc = fma(w[t][j], y[slot(t,j)][h], acc)
 *              for j = 0..k-1 in order.  Must not overlap y.
 *   stream     HIP stream
 */
MOE_API int moe_combine(const uint16_t *y, int32_t E, int32_t capacity, int32_t H,
                        const int32_t *token_slot, const float *topk_w, int64_t T, int32_t k,
                        uint16_t *out, hipStream_t stream);

/*
 * moe_combine_residual_rmsnorm -- moe_combine with its epilogue fused: the
 * residual add and the next module's RMSNorm.
 *
 * "How GPUs Talk to Each Other During LLM Inference", section 5: right
 * after a sum, the result is added to the residual stream, the updated
 * stream is stored, and it is normalised (x * rsqrt(mean of squares over the
 * token + eps) * gamma) before anything else is written -- one pass instead
 * of three kernels that each read and write the same tensor.  Here the sum
 * is combine's weighted sum.
 *
 *   y, E, capacity, token_slot, topk_w, T, k: as for moe_combine
 *   H             hidden size, multiple of 8, <= MOE_MAX_NORM_HIDDEN
 *   residual      (device, in)  bf16 [T][H], 16 B aligned
 *   gamma         (device, in)  bf16 [H] RMSNorm weight, 16 B aligned
 *   eps           >= 0, finite
 *   residual_out  (device, out) bf16 [T][H], 16 B aligned: bf16 RNE of
 *                 r = acc + residual (one fp32 addition; acc is exactly
 *                 moe_combine's fp32 accumulator).  May be `residual`
 *                 itself (in-place update); must not overlap it otherwise.
 *   normed_out    (device, out) bf16 [T][H], 16 B aligned: (r * inv) *
 *                 gamma with inv = 1 / sqrt(sum(r^2)/H + eps), from the
 *                 unrounded fp32 r, evaluated in double and rounded to bf16
 *                 (nearest even) in one step; no underflow or overflow for
 *                 any finite row.  The sum of squares runs in a fixed order
 *                 per launch shape, so results are identical run to run.
 *                 Must not overlap any other buffer.  With eps = 0 an
 *                 all-zero row gives NaN.
 *   stream        HIP stream
 * No output may overlap an input (y, token_slot, topk_w, residual except as
 * above, gamma) or another output: MOE_ERR_INVALID.  T = 0 enqueues nothing.
 */
MOE_API int moe_combine_residual_rmsnorm(const uint16_t *y, int32_t E, int32_t capacity, int32_t H,
                                         const int32_t *token_slot, const float *topk_w, int64_t T, int32_t k,
                                         const uint16_t *residual, const uint16_t *gamma, float eps,
                                         uint16_t *residual_out, uint16_t *normed_out, hipStream_t stream);

/*
 * moe_combine_residual_rmsnorm_fp8 -- the fused epilogue above, with the
 * normalised rows also re-quantised for an fp8 consumer (the next layer's
 * fp8 GEMM).
 *
 * Handbook "NVSHMEM and DeepEP", "High-throughput mode": activations travel
 * as FP8 with one fp32 scale per 128 elements.  The encoding is
 * moe_dispatch's MOE_DTYPE_FP8_E4M3 one, applied to the bf16 normalised
 * values: per 128-element block sc = amax / 448 (1 for an all-zero block)
 * and each code is the E4M3 encoding (nearest even, saturating) of x / sc.
 *
 *   all arguments as for moe_combine_residual_rmsnorm, except
 *   H             also a multiple of 128 (else MOE_ERR_UNSUPPORTED)
 *   normed_out    (device, out, may be NULL) the bf16 normalised rows; the
 *                 codes are those of these values whether or not they are
 *                 stored
 *   normed_q      (device, out) uint8 [T][H] E4M3 codes, 8 B aligned
 *   normed_scales (device, out) float [T][H/128] block scales, 4 B aligned
 */
MOE_API int moe_combine_residual_rmsnorm_fp8(const uint16_t *y, int32_t E, int32_t capacity, int32_t H,
                                             const int32_t *token_slot, const float *topk_w, int64_t T, int32_t k,
                                             const uint16_t *residual, const uint16_t *gamma, float eps,
                                             uint16_t *residual_out, uint16_t *normed_out, uint8_t *normed_q,
                                             float *normed_scales, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
