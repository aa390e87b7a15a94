"""libqmm for MI355X: matrix multiplies whose weights are block-quantized 4/6-bit
codes dequantized inside hand-written gfx950 HIP kernels against bfloat16
activations.  The C ABI is include/qmm.h; this package is its ctypes binding.
"""

from .qmm import (AFFINE4_G64, BF16, F32, FORMATS, MXFP4, NVFP4, Q6_K, PreparedGemv, QmmError,  # noqa: F401
                  Weight, bench_mfma_peak, bench_stream_read, dequant, gemm, gemv, moe, moe_from_logits,
                  moe_noalloc, moe_router, moe_workspace_layout,
                  moe_workspace_size, gemv_workspace_size, lib_handle, new_workspace,
                  workspace_init, prepare_gemm, prepare_moe, quant_mxfp4, gemm_w4a4,
                  gemm_w4a4_workspace_size, prepare_gemm_w4a4, hadamard_prepare,
                  hadamard_finish, gemv_hadamard)
