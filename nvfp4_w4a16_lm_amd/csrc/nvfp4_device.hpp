// Device-side helpers shared by the NVFP4 kernels (gfx950 only).
//
// Formats (vLLM API docs, quantization.online.lm_head, _quantize_nvfp4):
//   E2M1 code: bit 3 = sign, bits 0-2 index the magnitudes {0,.5,1,1.5,2,3,4,6};
//   two codes per byte, the even-k code in the low nibble;
//   block scale: float8_e4m3fn (1-4-3, bias 7, no infinity, 0x7F = NaN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 16;          // weights per E4M3 block scale
constexpr float kE2m1Max = 6.0f;    // largest E2M1 magnitude
constexpr float kE4m3Max = 448.0f;  // largest finite float8_e4m3fn

// 16-byte load that bypasses cache allocation priority (streamed once).
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Max of two pairs of unsigned 16-bit lanes.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 r = __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b));
  return __builtin_bit_cast(uint32_t, r);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-negative float u <= 448 -> E4M3 byte (nearest, ties to even mantissa);
// also returns the byte's value.  Subnormal range (u < 2^-6): multiples of
// 2^-9; rintf rounds half to even.  Normal range: round the fp32 mantissa to
// 3 bits at bit 20 with the nearest-even bias; a carry moves to the exponent.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float u, float* value) {
  const float m = rintf(u * 512.0f);
  const uint32_t ub = __float_as_uint(u);
  const uint32_t r = (ub + 0x7FFFFu + ((ub >> 20) & 1u)) >> 20;
  const bool sub = u < 0.015625f;
  *value = sub ? m * 0.001953125f : __uint_as_float(r << 20);
  return sub ? (uint32_t)m : r - (120u << 3);
}

// E4M3 byte -> float (exact).  Sign honoured; 0x7F/0xFF (NaN) are not produced
// by the quantizer and are outside the contract of the GEMM.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t mag = b & 0x7Fu;
  const float sub = (float)(mag & 7u) * 0.001953125f;
  const float nrm = __uint_as_float((mag + 960u) << 20);
  const float v = (mag < 8u) ? sub : nrm;
  return (b & 0x80u) ? -v : v;
}

// E2M1 magnitude code of 0 <= a <= 6: nearest grid value, ties to the even code.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// 4-bit code -> its value times the block scale s, as fp32 (exact: at most
// 2 significant bits times at most 4).
__device__ __forceinline__ float e2m1_scaled(uint32_t c, float s) {
  const uint32_t mag = c & 7u;
  const float big = __uint_as_float((mag << 22) + 0x3F000000u);  // mag >= 2: 2^(e-1)(1+m/2)
  const float small = (mag == 1u) ? 0.5f : 0.0f;
  float v = (mag >= 2u) ? big : small;
  v = __uint_as_float(__float_as_uint(v) ^ ((c & 8u) << 28));
  return v * s;
}

// Eight codes (one 32-bit word, code i in bits 4i..4i+3) -> eight bf16 values
// of code * s.  The products are exact in bf16, so taking the upper 16 bits of
// the fp32 product is exact.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = __float_as_uint(e2m1_scaled((w >> (8 * j)) & 0xFu, s));
    const uint32_t hi = __float_as_uint(e2m1_scaled((w >> (8 * j + 4)) & 0xFu, s));
    o[j] = (lo >> 16) | (hi & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8, o);
}

}  // namespace nvfp4
