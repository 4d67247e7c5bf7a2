// moe_api.cpp -- the C ABI of libmoe_route.so: argument checks, then the
// kernel launches.  The operations and their contracts are documented in
// include/moe_route.h.
#include "moe_route.h"

#include <limits.h>

#include "kernels.hpp"

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Do the byte ranges [a, a + na) and [b, b + nb) overlap?
bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// A buffer as a byte range; n == 0 marks one that is absent or unused.
struct Region {
    const void *p;
    uint64_t n;
};

// Does an output overlap an input or another output?  (Inputs may share
// memory with each other.)
template <int NO, int NI>
bool any_overlap(const Region (&out)[NO], const Region (&in)[NI])
{
    for (int i = 0; i < NO; ++i) {
        if (!out[i].n)
            continue;
        for (int j = 0; j < NI; ++j)
            if (in[j].n && overlaps(out[i].p, out[i].n, in[j].p, in[j].n))
                return true;
        for (int j = i + 1; j < NO; ++j)
            if (out[j].n && overlaps(out[i].p, out[i].n, out[j].p, out[j].n))
                return true;
    }
    return false;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Shared checks of E and k.
int check_ek(int32_t E, int32_t k)
{
    if (E < 1 || k < 1 || k > E)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Checks shared by both dispatch layouts.  Exactly one of expert_counts
// (fixed slots of `capacity` rows) and expert_offsets (packed) is used.
int dispatch_checked(const uint16_t *x, int64_t T, int32_t H, const int32_t *topk_idx, int32_t E, int32_t k,
                     int32_t capacity, int32_t out_dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                     int32_t *expert_counts, int32_t *expert_offsets, int32_t *token_slot, void *workspace,
                     size_t workspace_bytes, hipStream_t stream)
{
    if (T < 0 || H < 1)
        return MOE_ERR_INVALID;
    int rc = check_ek(E, k);
    if (rc != MOE_OK)
        return rc;
    if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3)
        return MOE_ERR_INVALID;
    if (H % 8 != 0 || (out_dtype == MOE_DTYPE_FP8_E4M3 && H % 128 != 0))
        return MOE_ERR_UNSUPPORTED;
    if (T > MOE_MAX_TOKENS)
        return MOE_ERR_UNSUPPORTED;
    int32_t *per_expert = expert_offsets ? expert_offsets : expert_counts;
    if (!per_expert || !aligned(per_expert, 4))
        return MOE_ERR_INVALID;
    if (T > 0) {
        if (!x || !topk_idx || !recv_x || !recv_src || !token_slot)
            return MOE_ERR_INVALID;
        if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 4) || !aligned(recv_src, 4) ||
            !aligned(token_slot, 4))
            return MOE_ERR_INVALID;
        if (out_dtype == MOE_DTYPE_FP8_E4M3 && (!recv_scales || !aligned(recv_scales, 4)))
            return MOE_ERR_INVALID;
    }
    if (out_dtype == MOE_DTYPE_BF16 && recv_scales)
        return MOE_ERR_INVALID;
    const size_t need = moe::dispatch_workspace_bytes(T, E, k);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return MOE_ERR_WORKSPACE;
    if (T > 0) {
        const uint64_t rows = expert_offsets ? (uint64_t)T * k : (uint64_t)E * capacity;
        const uint64_t row_bytes = out_dtype == MOE_DTYPE_FP8_E4M3 ? (uint64_t)H : 2 * (uint64_t)H;
        const Region in[] = {{x, (uint64_t)T * H * 2}, {topk_idx, (uint64_t)T * k * 4}};
        const Region out[] = {{recv_x, rows * row_bytes},
                              {recv_scales, recv_scales ? rows * (H / 128) * 4 : 0},
                              {recv_src, rows * 4},
                              {per_expert, (uint64_t)(expert_offsets ? E + 1 : E) * 4},
                              {token_slot, (uint64_t)T * k * 4},
                              {workspace, need}};
        if (any_overlap(out, in))
            return MOE_ERR_INVALID;
    }
    if (!moe::dispatch_grid_fits(T, H, k, out_dtype))
        return MOE_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return from_hip(moe::launch_dispatch(x, T, H, topk_idx, E, k, capacity, out_dtype, recv_x, recv_scales,
                                         recv_src, expert_counts, expert_offsets, token_slot, workspace, stream));
}

}  // namespace

extern "C" {

MOE_API const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "batch needs more workspace than the static scratch (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

MOE_API int moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_idx,
                           float *topk_w, hipStream_t stream)
{
    if (T < 0)
        return MOE_ERR_INVALID;
    int rc = check_ek(E, k);
    if (rc != MOE_OK)
        return rc;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID;
    if (T > MOE_MAX_TOKENS)
        return MOE_ERR_UNSUPPORTED;
    const Region in[] = {{logits, (uint64_t)T * E * 4}};
    const Region out[] = {{topk_idx, (uint64_t)T * k * 4}, {topk_w, (uint64_t)T * k * 4}};
    if (any_overlap(out, in))
        return MOE_ERR_INVALID;
    (void)hipGetLastError();
    return from_hip(moe::launch_route_topk(logits, T, E, k, topk_idx, topk_w, stream));
}

MOE_API int moe_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t k, int32_t n_groups,
                                   int32_t topk_groups, int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    if (T < 0)
        return MOE_ERR_INVALID;
    int rc = check_ek(E, k);
    if (rc != MOE_OK)
        return rc;
    if (n_groups < 1 || E % n_groups != 0 || E / n_groups < 2 || topk_groups < 1 || topk_groups > n_groups ||
        (int64_t)topk_groups * (E / n_groups) < k)
        return MOE_ERR_INVALID;
    if (n_groups > MOE_MAX_GROUPS)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID;
    if (T > MOE_MAX_TOKENS)
        return MOE_ERR_UNSUPPORTED;
    const Region in[] = {{logits, (uint64_t)T * E * 4}};
    const Region out[] = {{topk_idx, (uint64_t)T * k * 4}, {topk_w, (uint64_t)T * k * 4}};
    if (any_overlap(out, in))
        return MOE_ERR_INVALID;
    (void)hipGetLastError();
    return from_hip(moe::launch_route_topk_grouped(logits, T, E, k, n_groups, topk_groups, topk_idx, topk_w, stream));
}

MOE_API size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k)
{
    if (T < 0 || E < 1 || k < 1 || E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)
        return 0;
    return moe::dispatch_workspace_bytes(T, E, k);
}

MOE_API int moe_dispatch(const uint16_t *x, int64_t T, int32_t H, const int32_t *topk_idx, int32_t E, int32_t k,
                         int32_t capacity, int32_t out_dtype, void *recv_x, float *recv_scales,
                         int32_t *recv_src, int32_t *expert_counts, int32_t *token_slot, void *workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    if (capacity < 1)
        return MOE_ERR_INVALID;
    if ((int64_t)E * capacity > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    return dispatch_checked(x, T, H, topk_idx, E, k, capacity, out_dtype, recv_x, recv_scales, recv_src,
                            expert_counts, nullptr, token_slot, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Shared checks of moe_route_dispatch (expert_offsets == NULL, fixed slots)
// and moe_route_dispatch_packed (capacity unused).
int route_dispatch_checked(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x, int32_t H,
                           int32_t capacity, int32_t out_dtype, int32_t *topk_idx, float *topk_w, void *recv_x,
                           float *recv_scales, int32_t *recv_src, int32_t *expert_counts, int32_t *expert_offsets,
                           int32_t *token_slot, void *workspace, size_t workspace_bytes, hipStream_t stream,
                           bool noalloc = false)
{
    if (T < 0 || H < 1 || capacity < 1)
        return MOE_ERR_INVALID;
    int rc = check_ek(E, k);
    if (rc != MOE_OK)
        return rc;
    if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3)
        return MOE_ERR_INVALID;
    if (H % 8 != 0 || (out_dtype == MOE_DTYPE_FP8_E4M3 && H % 128 != 0))
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)E * capacity > INT32_MAX || T > MOE_MAX_TOKENS || T * (int64_t)k > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    int32_t *per_expert = expert_offsets ? expert_offsets : expert_counts;
    if (!per_expert || !aligned(per_expert, 4))
        return MOE_ERR_INVALID;
    if (T > 0) {
        if (!logits || !x || !topk_idx || !topk_w || !recv_x || !recv_src || !token_slot)
            return MOE_ERR_INVALID;
        if (!aligned(logits, 4) || !aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 4) ||
            !aligned(topk_w, 4) || !aligned(recv_src, 4) || !aligned(token_slot, 4))
            return MOE_ERR_INVALID;
        if (out_dtype == MOE_DTYPE_FP8_E4M3 && (!recv_scales || !aligned(recv_scales, 4)))
            return MOE_ERR_INVALID;
    }
    if (out_dtype == MOE_DTYPE_BF16 && recv_scales)
        return MOE_ERR_INVALID;
    const size_t need = moe::dispatch_workspace_bytes(T, E, k);
    if (noalloc) {   // the library's static array stands in for the workspace
        if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
            return MOE_ERR_SCRATCH;
        if (moe::noalloc_scratch(&workspace) != hipSuccess)
            return MOE_ERR_HIP;
        workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return MOE_ERR_WORKSPACE;
    if (T > 0) {
        const uint64_t rows = expert_offsets ? (uint64_t)T * k : (uint64_t)E * capacity;
        const uint64_t row_bytes = out_dtype == MOE_DTYPE_FP8_E4M3 ? (uint64_t)H : 2 * (uint64_t)H;
        const Region in[] = {{logits, (uint64_t)T * E * 4}, {x, (uint64_t)T * H * 2}};
        const Region out[] = {{topk_idx, (uint64_t)T * k * 4},
                              {topk_w, (uint64_t)T * k * 4},
                              {recv_x, rows * row_bytes},
                              {recv_scales, recv_scales ? rows * (H / 128) * 4 : 0},
                              {recv_src, rows * 4},
                              {per_expert, (uint64_t)(expert_offsets ? E + 1 : E) * 4},
                              {token_slot, (uint64_t)T * k * 4},
                              {workspace, need}};
        if (any_overlap(out, in))
            return MOE_ERR_INVALID;
    }
    if (!moe::dispatch_grid_fits(T, H, k, out_dtype))
        return MOE_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return from_hip(moe::launch_route_dispatch(logits, T, E, k, x, H, capacity, out_dtype, topk_idx, topk_w, recv_x,
                                               recv_scales, recv_src, expert_counts, expert_offsets, token_slot,
                                               workspace, stream));
}

}  // namespace

extern "C" {

MOE_API int moe_route_dispatch(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x, int32_t H,
                               int32_t capacity, int32_t out_dtype, int32_t *topk_idx, float *topk_w, void *recv_x,
                               float *recv_scales, int32_t *recv_src, int32_t *expert_counts, int32_t *token_slot,
                               void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return route_dispatch_checked(logits, T, E, k, x, H, capacity, out_dtype, topk_idx, topk_w, recv_x, recv_scales,
                                  recv_src, expert_counts, nullptr, token_slot, workspace, workspace_bytes, stream);
}

MOE_API int moe_route_dispatch_noalloc(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x,
                                       int32_t H, int32_t capacity, int32_t out_dtype, int32_t *topk_idx,
                                       float *topk_w, void *recv_x, float *recv_scales, int32_t *recv_src,
                                       int32_t *expert_counts, int32_t *token_slot, hipStream_t stream)
{
    return route_dispatch_checked(logits, T, E, k, x, H, capacity, out_dtype, topk_idx, topk_w, recv_x, recv_scales,
                                  recv_src, expert_counts, nullptr, token_slot, nullptr, 0, stream, true);
}

MOE_API int moe_route_dispatch_packed(const float *logits, int64_t T, int32_t E, int32_t k, const uint16_t *x,
                                      int32_t H, int32_t out_dtype, int32_t *topk_idx, float *topk_w, void *recv_x,
                                      float *recv_scales, int32_t *recv_src, int32_t *expert_offsets,
                                      int32_t *token_slot, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    return route_dispatch_checked(logits, T, E, k, x, H, 1, out_dtype, topk_idx, topk_w, recv_x, recv_scales,
                                  recv_src, nullptr, expert_offsets, token_slot, workspace, workspace_bytes, stream);
}

MOE_API int moe_dispatch_packed(const uint16_t *x, int64_t T, int32_t H, const int32_t *topk_idx, int32_t E,
                                int32_t k, int32_t out_dtype, void *recv_x, float *recv_scales, int32_t *recv_src,
                                int32_t *expert_offsets, int32_t *token_slot, void *workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    if (T * (int64_t)(k > 0 ? k : 1) > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    return dispatch_checked(x, T, H, topk_idx, E, k, 0, out_dtype, recv_x, recv_scales, recv_src, nullptr,
                            expert_offsets, token_slot, workspace, workspace_bytes, stream);
}

namespace {

int combine_checked(const uint16_t *y, int32_t E, int32_t capacity, int32_t H, const int32_t *token_slot,
                    const float *topk_w, int64_t T, int32_t k, uint16_t *out, hipStream_t stream)
{
    if (T < 0 || H < 1 || capacity < 1 || E < 1 || k < 1)
        return MOE_ERR_INVALID;
    if (k > MOE_MAX_TOPK || H % 8 != 0)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)E * capacity > INT32_MAX || T > MOE_MAX_TOKENS)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!y || !token_slot || !topk_w || !out)
        return MOE_ERR_INVALID;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(token_slot, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID;
    const Region in[] = {{y, (uint64_t)E * capacity * H * 2},
                         {token_slot, (uint64_t)T * k * 4},
                         {topk_w, (uint64_t)T * k * 4}};
    const Region out_r[] = {{out, (uint64_t)T * H * 2}};
    if (any_overlap(out_r, in))
        return MOE_ERR_INVALID;
    if (!moe::combine_grid_fits(T, H, k))
        return MOE_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return from_hip(
        moe::launch_combine(y, (int64_t)E * capacity, H, token_slot, topk_w, T, k, out, stream));
}

}  // namespace

MOE_API int moe_combine(const uint16_t *y, int32_t E, int32_t capacity, int32_t H, const int32_t *token_slot,
                        const float *topk_w, int64_t T, int32_t k, uint16_t *out, hipStream_t stream)
{
    return combine_checked(y, E, capacity, H, token_slot, topk_w, T, k, out, stream);
}

}  // extern "C"

namespace {

int norm_checked(const uint16_t *y, int32_t E, int32_t capacity, int32_t H, const int32_t *token_slot,
                 const float *topk_w, int64_t T, int32_t k, const uint16_t *residual, const uint16_t *gamma, float eps,
                 uint16_t *residual_out, uint16_t *normed_out, bool q, uint8_t *normed_q, float *normed_scales,
                 hipStream_t stream)
{
    if (T < 0 || H < 1 || capacity < 1 || E < 1 || k < 1 || !(eps >= 0.0f) || !(eps <= 3.4e38f))
        return MOE_ERR_INVALID;
    if (k > MOE_MAX_TOPK || H % 8 != 0 || H > MOE_MAX_NORM_HIDDEN || (q && H % 128 != 0))
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)E * capacity > INT32_MAX || T > MOE_MAX_TOKENS)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!y || !token_slot || !topk_w || !residual || !gamma || !residual_out || (!q && !normed_out))
        return MOE_ERR_INVALID;
    if (q && (!normed_q || !normed_scales || !aligned(normed_q, 8) || !aligned(normed_scales, 4)))
        return MOE_ERR_INVALID;
    if (!aligned(y, 16) || !aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) ||
        (normed_out && !aligned(normed_out, 16)) || !aligned(token_slot, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID;
    const uint64_t ybytes = (uint64_t)E * capacity * H * 2, row_bytes = (uint64_t)T * H * 2;
    // outputs must not overlap the inputs or each other; residual_out may be
    // residual itself (an in-place update of the residual stream)
    const Region in[] = {{y, ybytes},
                         {residual, residual_out == residual ? 0 : row_bytes},
                         {gamma, 2 * (uint64_t)H},
                         {token_slot, (uint64_t)T * k * 4},
                         {topk_w, (uint64_t)T * k * 4}};
    const Region out[] = {{residual_out, row_bytes},
                          {normed_out, normed_out ? row_bytes : 0},
                          {normed_q, q ? (uint64_t)T * H : 0},
                          {normed_scales, q ? (uint64_t)T * (H / 128) * 4 : 0}};
    if (any_overlap(out, in))
        return MOE_ERR_INVALID;
    (void)hipGetLastError();
    return from_hip(moe::launch_combine_rmsnorm(y, (int64_t)E * capacity, H, token_slot, topk_w, T, k, residual,
                                                gamma, eps, residual_out, normed_out, normed_q, normed_scales,
                                                stream));
}

}  // namespace

extern "C" {

MOE_API int moe_combine_residual_rmsnorm(const uint16_t *y, int32_t E, int32_t capacity, int32_t H,
                                         const int32_t *token_slot, const float *topk_w, int64_t T, int32_t k,
                                         const uint16_t *residual, const uint16_t *gamma, float eps,
                                         uint16_t *residual_out, uint16_t *normed_out, hipStream_t stream)
{
    return norm_checked(y, E, capacity, H, token_slot, topk_w, T, k, residual, gamma, eps, residual_out,
                        normed_out, false, nullptr, nullptr, stream);
}

MOE_API int moe_combine_residual_rmsnorm_fp8(const uint16_t *y, int32_t E, int32_t capacity, int32_t H,
                                             const int32_t *token_slot, const float *topk_w, int64_t T, int32_t k,
                                             const uint16_t *residual, const uint16_t *gamma, float eps,
                                             uint16_t *residual_out, uint16_t *normed_out, uint8_t *normed_q,
                                             float *normed_scales, hipStream_t stream)
{
    return norm_checked(y, E, capacity, H, token_slot, topk_w, T, k, residual, gamma, eps, residual_out,
                        normed_out, true, normed_q, normed_scales, stream);
}

}  // extern "C"
