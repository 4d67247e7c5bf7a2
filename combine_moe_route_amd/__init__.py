"""MoE token routing, dispatch and combine for AMD Instinct MI355X (gfx950).

The computation lives in libmoe_route.so (hand-written HIP kernels behind a
C ABI, include/moe_route.h); this package is its build script and a thin
ctypes binding with the same entry-point names.
"""
from .binding import (  # noqa: F401
    MOE_DTYPE_BF16,
    MOE_DTYPE_FP8_E4M3,
    MOE_MAX_EXPERTS,
    MOE_MAX_TOPK,
    MOE_NOALLOC_SCRATCH_BYTES,
    DispatchBuffers,
    HipEvents,
    MoeError,
    PackedBuffers,
    PreparedStep,
    load,
    moe_combine,
    moe_combine_residual_rmsnorm,
    moe_combine_residual_rmsnorm_fp8,
    moe_dispatch,
    moe_dispatch_packed,
    moe_dispatch_workspace_bytes,
    moe_route_dispatch,
    moe_route_dispatch_noalloc,
    moe_route_dispatch_packed,
    moe_route_topk,
    moe_route_topk_grouped,
    moe_status_string,
)
from .build import LIB_PATH, build  # noqa: F401
