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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 16;          // weights per E4M3 block scale
constexpr float kE2m1Max = 6.0f;    // largest E2M1 magnitude
constexpr float kE4m3Max = 448.0f;  // largest finite float8_e4m3fn

// 16-byte load that bypasses cache allocation priority (streamed once).
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Sum over the 16 lanes of each DPP row (quad swaps, then half-row and row mirrors).
__device__ __forceinline__ float dpp_row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row mirror
  return v;
}

// Four per-lane partials (rows 0..3 of a batch) -> full wavefront sums, with
// row i ending up in every lane whose bits 5,4 equal (i >> 1, i & 1).
__device__ __forceinline__ float wave_sum4(const float p[4], int lane) {
  const bool h5 = lane & 32, h4 = lane & 16;
  const float s0 = h5 ? p[0] : p[2], k0 = h5 ? p[2] : p[0];
  const float s1 = h5 ? p[1] : p[3], k1 = h5 ? p[3] : p[1];
  const float w0 = k0 + __shfl_xor(s0, 32, 64);
  const float w1 = k1 + __shfl_xor(s1, 32, 64);
  const float s = h4 ? w0 : w1, k = h4 ? w1 : w0;
  return dpp_row_sum(k + __shfl_xor(s, 16, 64));
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

// Two floats -> two E2M1 codes in byte SEL of `old` (gfx950 converter, scale 1).
// The converter rounds the magnitude to nearest with ties to the even code and
// saturates at 6; it copies the sign bit of its input even when the magnitude
// rounds to zero, which fix_zero_signs() undoes.
#define NVFP4_CVT_PK_FP4(old, a, b, SEL) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (SEL))

// Clear the sign bit of every nibble whose magnitude bits are zero, so zero is
// always code 0x0: adding 7 to a 3-bit magnitude sets bit 3 exactly when the
// magnitude is nonzero, with no carry into the next nibble.
__device__ __forceinline__ uint32_t fix_zero_signs(uint32_t w) {
  const uint32_t mag = w & 0x77777777u;
  const uint32_t nonzero = (mag + 0x77777777u) & 0x88888888u;
  return mag | (w & nonzero);
}

// E4M3 byte SEL of a 32-bit word -> float (gfx950 converter, OCP e4m3fn).
#define NVFP4_E4M3_TO_F32(word, SEL) __builtin_amdgcn_cvt_f32_fp8((int)(word), (SEL))

// E4M3 bytes 2 SEL and 2 SEL + 1 of a 32-bit word -> a pair of bf16 (gfx950
// converter with scale 1; every finite e4m3fn value is exact in bf16).
#define NVFP4_E4M3X2_TO_BF16(word, SEL) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((word), 1.0f, (SEL))

// Byte j of `w` (two codes, the low nibble first) -> the two values
// code * s as a packed pair of bf16.  The converter gives the exact E2M1
// values as fp32; code * s has at most 6 significant bits, so the fp32
// product is exact and its upper half is the exact bf16.
#define NVFP4_DEQ_PAIR(w, s, SEL)                                                         \
  ([&]() {                                                                                \
    const f32x2 d_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((w), 1.0f, (SEL));        \
    return __builtin_amdgcn_perm(__float_as_uint(d_[1] * (s)), __float_as_uint(d_[0] * (s)), \
                                 0x07060302u);                                            \
  }())

// Eight codes (one 32-bit word, code i in bits 4i..4i+3) -> eight bf16 values
// of code * s.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  u32x4 o;
  o[0] = NVFP4_DEQ_PAIR(w, s, 0);
  o[1] = NVFP4_DEQ_PAIR(w, s, 1);
  o[2] = NVFP4_DEQ_PAIR(w, s, 2);
  o[3] = NVFP4_DEQ_PAIR(w, s, 3);
  return __builtin_bit_cast(bf16x8, o);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// E4M3 scale s (as fp32) = e2 * mu: e2 = 2^e (its exponent field), mu in
// [1, 2) (its significand, 3 fraction bits) as an f16 pair; s = 0 gives mu 0.
// The fp4 converters below apply only the exponent of their fp32 scale, so
// they take e2 and the mantissa mu is applied separately.
__device__ __forceinline__ void split_scale(float s, float* e2, f16x2* mu) {
  const uint32_t b = __float_as_uint(s);
  *e2 = __uint_as_float(b & 0x7F800000u);
  const _Float16 m = (s == 0.0f) ? (_Float16)0.0f : (_Float16)__uint_as_float((b & 0x007FFFFFu) | 0x3F800000u);
  *mu = f16x2{m, m};
}

// Codes 0..7 of w (low nibble first) times e2 * mu, exact in f16: the
// converter applies e2 exactly and code * e2 * mu has at most 6 significant
// bits within [2^-10, 2688].
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, float e2, f16x2 mu) {
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e2, 0) * mu;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e2, 1) * mu;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e2, 2) * mu;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, e2, 3) * mu;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// E4M3 block scale s (fp32) -> the mantissa mu = s / 2^e as an f16 pair, for
// dequant8_f16(w, s, mu): the fp4 converter takes s itself as its scale and
// applies only its exponent.  mu = 1.f with f the top 10 fraction bits of s
// (an E4M3 value has at most 3, so mu is exact).  For s = 0 the converter's
// scale is 2^-127, every code converts to a signed f16 zero, and mu = 1
// leaves it zero.
__device__ __forceinline__ f16x2 scale_mantissa_f16(float s) {
  const uint32_t h = 0x3C00u | ((__float_as_uint(s) >> 13) & 0x3FFu);
  return __builtin_bit_cast(f16x2, h | (h << 16));
}

}  // namespace nvfp4
