"""MI355X (gfx950) NVFP4 block-scaled GEMM: y = x . W^T with E2M1 operands,
E4M3FN scales per 16 elements and fp32 per-tensor global scales.

The computation lives in ``libnvfp4.so`` (HIP kernels + C ABI, declared in
``include/nvfp4.h``); this package only marshals torch tensors into it.
"""
from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, NVFP4_BF16, NVFP4_GROUPED_MAX_PROBLEMS, GroupedProblem, NVFP4_ERR_HIP, NVFP4_ERR_INVALID_ARG,
    NVFP4_ERR_UNSUPPORTED, NVFP4_F32, NVFP4_GLOBAL_SCALE_GIVEN, NVFP4_OK, Nvfp4Error,
    Packed, load, nvfp4_gemm, nvfp4_gemm_nvfp4_out, nvfp4_gemm_nvfp4_out_raw, nvfp4_gemm_raw,
    nvfp4_grouped_gemm, nvfp4_grouped_gemm_gather_raw, nvfp4_grouped_gemm_multi,
    nvfp4_grouped_gemm_multi_raw, nvfp4_grouped_gemm_raw, nvfp4_mxfp4_gemm,
    nvfp4_mxfp4_gemm_raw, nvfp4_mxfp4_quantize, nvfp4_mxfp4_quantize_raw,
    nvfp4_quantize, nvfp4_quantize_noalloc_raw, nvfp4_quantize_raw, nvfp4_quantize_workspace_bytes,
)
