"""CPU oracle for the NVFP4 block-scaled GEMM (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the HIP library never does.
"""
from .nvfp4_ref import (  # noqa: F401
    E2M1_MAGNITUDES, E2M1_TABLE, E4M3_MAX, GLOBAL_DIVISOR, REL_TOL,
    check_gemm, dequantize_ref, e2m1_decode, e4m3_decode, gemm_ref,
    global_scale_ref, grouped_gemm_ref, pack_nibbles, quantize_ref,
    tolerance, ulp_bf16, unpack_nibbles,
)
from .mxfp4_ref import (  # noqa: F401
    MX_BLOCK, e8m0_decode, mxfp4_dequantize_ref, mxfp4_gemm_ref, mxfp4_quantize_ref,
)
