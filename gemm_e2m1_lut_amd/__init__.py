"""gemm_e2m1_lut_amd -- low-bit weight decoding inside memory-bound GEMV / small-batch GEMM
for AMD MI355X (gfx950).

The product is the C-ABI library libe2m1lut.so (include/e2m1lut.h), built from
the HIP sources in csrc/ by build.py. This package is its thin Python binding:
torch supplies device memory and streams; every step of every operation runs
in the library's kernels.

Operations: dequant_decode, dequant_gemv, dequant_gemv_grouped, dequant_gemm, ternary_gemv, ternary_gemm (+ workspace size),
ternary_wl_gemv, nvfp4_embedding_gather, mxfp4_moe_gemm (+
mxfp4_moe_workspace_size, and mxfp4_moe_gemm_noalloc for callers that cannot
allocate), nm_spmm (N:M structured-sparse weights), and the
encoders mxfp4_quantize, nvfp4_quantize.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION,
    DTYPE_BF16,
    DTYPE_F32,
    GEMV_MAX_BATCH,
    TERNARY_MAX_BATCH,
    LIB_PATH,
    E2M1Error,
    abi_version,
    dequant_decode,
    dequant_gemm,
    dequant_gemv,
    dequant_gemv_grouped,
    library_path,
    load_library,
    mxfp4_moe_gemm,
    mxfp4_moe_gemm_noalloc,
    MOE_NOALLOC_WORKSPACE_BYTES,
    mxfp4_moe_workspace_size,
    mxfp4_quantize,
    nvfp4_embedding_gather,
    nvfp4_quantize,
    nm_spmm,
    strerror,
    ternary_gemm,
    ternary_gemm_workspace_size,
    ternary_gemv,
    ternary_wl_gemv,
)
