// kernels.hpp -- host launchers of the library's kernels (internal).
// Arguments are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                             hipStream_t s);

// Router top-k for E <= 8 that also writes each expert's 32-token
// membership words: masks[e * ceil(T/32) + c].
hipError_t launch_route_topk_masks(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                                   uint32_t *masks, hipStream_t s);

// Router top-k for E > 8 that also writes the same 32-token membership
// words, a 16-token half per work-group (weights identical to
// launch_route_topk's).
hipError_t launch_route_topk_half_masks(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                                        uint32_t *masks, hipStream_t s);

// Route + dispatch in one call; the workspace is dispatch_workspace_bytes(T,
// E, k).  expert_offsets != NULL selects the packed layout (C and
// expert_counts unused), otherwise fixed slots of C rows per expert.
hipError_t launch_route_dispatch(const float *logits, int64_t T, int E, int k, const uint16_t *x, int H, int C,
                                 int dtype, int32_t *topk_idx, float *topk_w, void *recv_x, float *recv_scales,
                                 int32_t *recv_src, int32_t *expert_counts, int32_t *expert_offsets,
                                 int32_t *token_slot, void *workspace, hipStream_t s);

hipError_t launch_route_topk_grouped(const float *logits, int64_t T, int E, int k, int n_groups, int topk_groups,
                                     int32_t *idx, float *w, hipStream_t s);

size_t dispatch_workspace_bytes(int64_t T, int E, int k);

// Device address of the library's static scratch array on the current
// device (MOE_NOALLOC_SCRATCH_BYTES bytes, 256 B aligned), looked up on the
// first call per device.
hipError_t noalloc_scratch(void **out);

// Whether the pack (dispatch) or combine launch grid for this shape stays
// within one launch's 2^32 - 1 work-items (host-only, no HIP call).
bool dispatch_grid_fits(int64_t T, int H, int k, int dtype);
bool combine_grid_fits(int64_t T, int H, int k);

// expert_offsets != NULL selects the packed layout (C and expert_counts
// unused); otherwise fixed slots of C rows per expert.
hipError_t launch_dispatch(const uint16_t *x, int64_t T, int H, const int32_t *topk_idx, int E, int k, int C,
                           int dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                           int32_t *expert_counts, int32_t *expert_offsets, int32_t *token_slot, void *workspace,
                           hipStream_t s);

hipError_t launch_combine(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                          int64_t T, int k, uint16_t *out, hipStream_t s);

// combine + residual add + RMSNorm; residual_out may be residual (in place).
// normed_q != NULL adds the E4M3 codes [T][H] and per-128 scales [T][H/128]
// of the bf16 normalised rows (H % 128 == 0); normed_out may then be NULL.
hipError_t launch_combine_rmsnorm(const uint16_t *y, int64_t nrows, int H, const int32_t *token_slot, const float *w,
                                  int64_t T, int k, const uint16_t *residual, const uint16_t *gamma, float eps,
                                  uint16_t *residual_out, uint16_t *normed_out, uint8_t *normed_q,
                                  float *normed_scales, hipStream_t s);

}  // namespace moe
