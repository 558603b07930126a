"""Small-M BF16 x NVFP4 (W4A16) GEMV for AMD MI355X (gfx950).

The computation runs in the HIP library libw4a16_nvfp4_gemv.so (C ABI in
include/w4a16_nvfp4_gemv.h); this package only marshals torch tensors into
its entry points.
"""
from .ops import (  # noqa: F401
    W4A16Error, bf16_gemv, bf16_gemv_splitk, dequant_gemm, dequantize_rows, down_combine, gate_up, gemv_kernel_name,
    gemv_splitk_workspace, moe_down_combine, moe_gate_up, nvfp4_gemv, nvfp4_gemv_splitk, nvfp4_unswizzle_scales,
)
