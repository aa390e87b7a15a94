// SwiGLU's gate nonlinearity for the MoE gate/up epilogues (grouped GEMM and
// decode form), shared so that both forms give the same bits
// ("TurboEXL3" section 4.1: SwiGLU in 32-bit between gate/up and down).
#pragma once

#include <hip/hip_runtime.h>

namespace qmm {

// silu(g) = g / (1 + e^-g) in float32, e^-g as 2^(-g log2 e) on the hardware
// exp2 and the quotient by the hardware reciprocal, each within about one
// float32 ulp (h is rounded to bf16 after the product with u, 2^-9).  The
// limits hold: g -> -inf gives 2^+inf = inf, 1 / inf = 0, so silu -> 0 for
// finite g; g -> +inf gives g; NaN stays NaN.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace qmm
