// The EXL3 rotation stages around an inner product ("TurboEXL3" section 3.1:
// prepare scales the input by the input-channel vector and applies the
// Hadamard transform one 128-element block at a time; finish applies the
// transform to the output and then scales it by the output-channel vector;
// section 2.3: the transforms are sign-randomized Hadamard transforms in
// blocks of 128, and the two 16-bit channel vectors are the only scales).
//
// The transform is the orthonormal one, H_128 / sqrt(128) with H_128 in
// Sylvester's natural order (entry (i, j) = (-1)^popcount(i & j)); the random
// signs travel in the sign bits of the float16 channel scales.
//
// One wave per (row, block of 128): lane l holds elements l and l + 64.  The
// butterfly over index bit 6 pairs a lane's own two elements; those over bits
// 5 .. 0 pair lane l with lane l ^ span (cross-lane shuffles).  All sums are
// float32; the result is multiplied by float32(2^-3.5) at the end.  Prepare
// reads bf16 and writes bf16 (rounded to nearest even); finish reads float32
// and writes float32 or bf16.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

struct HadArgs {
  const void *in;         // bf16 (prepare) or float32 (finish) [rows][len]
  const uint16_t *scale;  // float16 [len] or null (all ones)
  void *out;              // bf16 (prepare), float32 or bf16 (finish) [rows][len]
  uint32_t units;         // rows * len / 128
  uint32_t blocks;        // len / 128
  uint32_t len;
  int out_bf16;
};

constexpr float kInvSqrt128 = 0.08838834764831844055f;  // 2^-3.5

template <bool PREPARE>
__global__ __launch_bounds__(256) void hadamard_kernel(HadArgs a) {
  const uint32_t unit = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (unit >= a.units) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const uint32_t row = unit / a.blocks, blk = unit - row * a.blocks;
  const size_t base = (size_t)row * a.len + (size_t)blk * 128;
  const uint32_t c0 = blk * 128u + (uint32_t)lane, c1 = c0 + 64u;  // channels
  float v0, v1;
  if constexpr (PREPARE) {
    const uint16_t *x = (const uint16_t *)a.in;
    v0 = bf_lo(x[base + lane]);
    v1 = bf_lo(x[base + lane + 64]);
    if (a.scale) {  // scale first, then transform
      v0 *= half_to_float(a.scale[c0]);
      v1 *= half_to_float(a.scale[c1]);
    }
  } else {
    const float *y = (const float *)a.in;
    v0 = y[base + lane];
    v1 = y[base + lane + 64];
  }
  // index bit 6: the lane's own pair
  {
    const float s = v0 + v1, d = v0 - v1;
    v0 = s;
    v1 = d;
  }
  // index bits 5 .. 0: lane l with lane l ^ span; the lane with the bit set
  // holds the difference (partner - own), the other the sum
#pragma unroll
  for (int span = 32; span >= 1; span >>= 1) {
    const float p0 = __shfl_xor(v0, span), p1 = __shfl_xor(v1, span);
    const bool upper = (lane & span) != 0;
    v0 = upper ? p0 - v0 : v0 + p0;
    v1 = upper ? p1 - v1 : v1 + p1;
  }
  v0 *= kInvSqrt128;
  v1 *= kInvSqrt128;
  if constexpr (!PREPARE) {
    if (a.scale) {  // transform first, then scale
      v0 *= half_to_float(a.scale[c0]);
      v1 *= half_to_float(a.scale[c1]);
    }
  }
  if (PREPARE || a.out_bf16) {
    uint16_t *o = (uint16_t *)a.out;
    o[base + lane] = (uint16_t)float_to_bf16(v0);
    o[base + lane + 64] = (uint16_t)float_to_bf16(v1);
  } else {
    float *o = (float *)a.out;
    o[base + lane] = v0;
    o[base + lane + 64] = v1;
  }
}

}  // namespace

hipError_t launch_hadamard(bool prepare, const void *in, int rows, int len, const void *scale,
                           void *out, int out_bf16, hipStream_t s) {
  HadArgs a;
  a.in = in;
  a.scale = (const uint16_t *)scale;
  a.out = out;
  a.blocks = (uint32_t)(len / 128);
  a.units = (uint32_t)rows * a.blocks;
  a.len = (uint32_t)len;
  a.out_bf16 = out_bf16;
  const dim3 grid((a.units + 3) / 4);
  if (prepare)
    hipLaunchKernelGGL(hadamard_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(hadamard_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qmm
