// qdequant: expand packed weights to float32 or bfloat16, one thread per run of
// 32 consecutive weights of a row (16 bytes of codes).  Every value is the exact
// weight rounded once to float32 ("TurboEXL3" section 2.1 for the three 4-bit
// formats, splash PR #19 "What changed" for Q6_K), then optionally rounded to
// nearest-even bfloat16.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

struct DequantArgs {
  const uint8_t *codes;
  const uint8_t *codes_hi;
  const uint8_t *scales;
  const uint8_t *scales2;
  const float *tensor_scale;
  void *out;
  int n, k;
  size_t chunks;  // batch * n * k / 32
};

template <int FMT>
__device__ __forceinline__ void decode32(const DequantArgs &a, size_t row, int kc, int e,
                                         float v[32]) {
  const size_t k = (size_t)a.k;
  const uint4 q = *(const uint4 *)(a.codes + row * (k / 2) + kc / 2);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  if constexpr (FMT == QMM_AFFINE4_G64) {
    const uint32_t sb = *(const uint32_t *)(a.scales + (row * (k / 64) + kc / 64) * 4);
    const float s = half_to_float(sb & 0xFFFFu), b = half_to_float(sb >> 16);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(s, (float)((w[i / 8] >> (4 * (i % 8))) & 15u), b);
  } else if constexpr (FMT == QMM_MXFP4 || FMT == QMM_NVFP4) {
    float s0, s1;
    if constexpr (FMT == QMM_MXFP4) {
      s0 = s1 = e8m0_to_float(a.scales[row * (k / 32) + kc / 32]);
    } else {
      s0 = e4m3_to_float(a.scales[row * (k / 16) + kc / 16]);
      s1 = e4m3_to_float(a.scales[row * (k / 16) + kc / 16 + 1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p[4] = {e2m1x2_to_bf16x2<0>(w[j]), e2m1x2_to_bf16x2<1>(w[j]),
                             e2m1x2_to_bf16x2<2>(w[j]), e2m1x2_to_bf16x2<3>(w[j])};
      const float sc = j < 2 ? s0 : s1;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[8 * j + 2 * b] = bf_lo(p[b]) * sc;
        v[8 * j + 2 * b + 1] = bf_hi(p[b]) * sc;
      }
    }
    if constexpr (FMT == QMM_NVFP4) {
      const float g = a.tensor_scale ? a.tensor_scale[e] : 1.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] *= g;
    }
  } else {  // Q6_K
    const uint2 h = *(const uint2 *)(a.codes_hi + row * (k / 4) + kc / 4);
    const uint32_t hw[2] = {h.x, h.y};
    const uint32_t sc2 = *(const uint16_t *)(a.scales + row * (k / 16) + kc / 16);
    const float d = half_to_float(*(const uint16_t *)(a.scales2 + (row * (k / 256) + kc / 256) * 2));
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t lo = (w[i / 8] >> (4 * (i % 8))) & 15u;
      const uint32_t hi = (hw[i / 16] >> (2 * (i % 16))) & 3u;
      const float dsc = d * (float)(int8_t)(sc2 >> (8 * (i / 16)));
      v[i] = dsc * (float)((int)(lo | (hi << 4)) - 32);
    }
  }
}

template <int FMT, int OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const size_t chunk = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (chunk >= a.chunks) return;
  const size_t per_row = (size_t)a.k / 32;
  const size_t row = chunk / per_row;  // row of the whole batch
  const int kc = (int)(chunk % per_row) * 32;
  const int e = (int)(row / (size_t)a.n);
  float v[32];
  decode32<FMT>(a, row, kc, e, v);
  if constexpr (OUT_BF16) {
    uint4 *o = (uint4 *)((uint16_t *)a.out + row * (size_t)a.k + kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 t;
      t.x = float_to_bf16(v[8 * j + 0]) | (float_to_bf16(v[8 * j + 1]) << 16);
      t.y = float_to_bf16(v[8 * j + 2]) | (float_to_bf16(v[8 * j + 3]) << 16);
      t.z = float_to_bf16(v[8 * j + 4]) | (float_to_bf16(v[8 * j + 5]) << 16);
      t.w = float_to_bf16(v[8 * j + 6]) | (float_to_bf16(v[8 * j + 7]) << 16);
      o[j] = t;
    }
  } else {
    float4 *o = (float4 *)((float *)a.out + row * (size_t)a.k + kc);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  }
}

template <int FMT>
hipError_t launch_fmt(const DequantArgs &a, int out_bf16, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.chunks + 255) / 256);
  if (out_bf16)
    hipLaunchKernelGGL((dequant_kernel<FMT, 1>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dequant_kernel<FMT, 0>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_dequant(const qmm_weight &w, int out_dtype, void *out, hipStream_t s) {
  DequantArgs a;
  a.codes = (const uint8_t *)w.codes;
  a.codes_hi = (const uint8_t *)w.codes_hi;
  a.scales = (const uint8_t *)w.scales;
  a.scales2 = (const uint8_t *)w.scales2;
  a.tensor_scale = w.tensor_scale;
  a.out = out;
  a.n = w.n;
  a.k = w.k;
  a.chunks = (size_t)w.batch * (size_t)w.n * (size_t)(w.k / 32);
  const int bf = out_dtype == QMM_BF16;
  switch (w.format) {
    case QMM_AFFINE4_G64: return launch_fmt<QMM_AFFINE4_G64>(a, bf, s);
    case QMM_MXFP4: return launch_fmt<QMM_MXFP4>(a, bf, s);
    case QMM_NVFP4: return launch_fmt<QMM_NVFP4>(a, bf, s);
    default: return launch_fmt<QMM_Q6_K>(a, bf, s);
  }
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, words);
  return hipGetLastError();
}

}  // namespace qmm
