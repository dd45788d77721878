"""libmxcast: bf16 -> MXFP8 casts, the 128x4 blocked e8m0 scale layout and
the row-wise and tensor-wise fp8 casts on AMD Instinct MI355X (gfx950), as hand-written HIP
kernels behind a C ABI (include/mxcast.h).  This package is the thin Python binding over that ABI;
the library is loaded on first use and its absence is an error."""
from ._binding import (  # noqa: F401
    MX_BLOCK,
    MX_MAX_GROUPS,
    MxError,
    LIB_PATH,
    lib,
    mx_blocked_bytes,
    mx_blocked_grouped_bytes,
    mx_cast_dim0_dim1,
    mx_cast_dim0_dim1_blocked,
    mx_cast_dim0_dim1_grouped_blocked,
    mx_cast_dim0_dim1_mgrouped,
    mx_cast_dim1_3d,
    mx_cast_dim1_3d_blocked,
    mx_gemm_mxfp8,
    mx_grouped_gemm_mxfp8,
    mx_kgrouped_gemm_mxfp8,
    mx_quantize_fp8_rowwise,
    mx_quantize_fp8_tensorwise,
    mx_quantize_fp8_tensorwise_noalloc,
    mx_scales_to_blocked,
    mx_scales_to_blocked_grouped,
    mx_tensorwise_workspace_bytes,
    status_string,
)
