// Device-side helpers shared by the libqmm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data that is read once (weights): non-temporal hint.
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bfloat16 pair (low half, high half) of a 32-bit word, widened to float.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float half_to_float(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// D = a.lo*b.lo + a.hi*b.hi + c, bfloat16 pairs, float32 accumulate
// (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two E2M1 codes (the byte BYTE of w: low nibble first) -> a bfloat16 pair,
// exactly (v_cvt_scalef32_pk_bf16_fp4 with a unit scale).
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, BYTE));
}

// E8M0 power-of-two scale -> float32 (2^(e-127); e = 0 is the subnormal 2^-127;
// 0xFF is NaN).
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
  e &= 0xFFu;
  uint32_t bits = e == 0 ? 0x00400000u : (e == 0xFFu ? 0x7FC00000u : e << 23);
  return __uint_as_float(bits);
}

// E4M3 (bias 7, subnormals, S.1111.111 = NaN) -> float32, exactly.
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  b &= 0xFFu;
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  if ((b & 0x7Fu) == 0x7Fu) v = __uint_as_float(0x7FC00000u);
  return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// The two E4M3 scales in the low 16 bits of w -> float32, with the gfx950
// FP8 conversion (OCP E4M3: bias 7, subnormals, S.1111.111 = NaN; a unit
// scale makes it exact).  It agrees with e4m3_to_float on all 256 codes.
__device__ __forceinline__ void e4m3x2_to_float(uint32_t w, float &s0, float &s1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  s0 = v.x;
  s1 = v.y;
}

// Buffer resource for raw buffer loads of `bytes` bytes at `base`; loads past
// the end return zeros (a null base with 0 bytes is a buffer that reads 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from buffer `r` (lane's byte offset voff + soff) straight
// to LDS at dst + 16 * lane, without passing through registers (buffer_load
// ... lds); dst must be wave-uniform.  The load counts in vmcnt like any other
// vector memory load.  (An ordinary function, so that host passes over kernel
// templates never see the LDS address space.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t voff,
                                                  uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt <= n and the other counters left free (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// float32 -> bfloat16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The orthonormal 128-point Hadamard transform H_128 / sqrt(128) (Sylvester's
// natural order, entry (i, j) = (-1)^popcount(i & j)) of one block held by a
// wave: lane l holds elements l (v0) and l + 64 (v1).  The butterfly over
// index bit 6 pairs a lane's own two elements; those over bits 5 .. 0 pair
// lane l with lane l ^ span, the lane with the bit set keeping the
// difference.  Float32 throughout, times 2^-3.5 at the end; every caller
// gets the same bits.
__device__ __forceinline__ void hadamard128_wave(float &v0, float &v1, int lane) {
  {
    const float s = v0 + v1, d = v0 - v1;
    v0 = s;
    v1 = d;
  }
#pragma unroll
  for (int span = 32; span >= 1; span >>= 1) {
    const float p0 = __shfl_xor(v0, span), p1 = __shfl_xor(v1, span);
    const bool upper = (lane & span) != 0;
    v0 = upper ? p0 - v0 : v0 + p0;
    v1 = upper ? p1 - v1 : v1 + p1;
  }
  constexpr float kInvSqrt128 = 0.08838834764831844055f;  // 2^-3.5
  v0 *= kInvSqrt128;
  v1 *= kInvSqrt128;
}

}  // namespace qmm
