// Test support (not part of the library): runs the exact device code the
// quantizer and the GEMM kernels use for the E2M1 encode step and for weight
// dequantization, over inputs the tests choose, so that they can be compared
// value by value with the CPU oracle.
//
// Encode (vLLM API docs, quantization.online.lm_head, _quantize_nvfp4: the
// E2M1 code table and the sign rule "values < 0"): NVFP4_CVT_PK_FP4 on pairs
// of fp32 values, then fix_zero_signs, as quant_pack_kernel applies them to
// q = w * r.
//
// Dequantize (E2M1 code * E4M3 block scale): the fp32 route (dequant8), the
// f16 route in both forms (split_scale or the scale itself +
// scale_mantissa_f16, then dequant8_f16) and the power-of-two bf16 converter
// the dot kernel feeds to v_dot2_f32_bf16.
//
// FP8 copy: the e4m3 -> bf16 pair converter (NVFP4_E4M3X2_TO_BF16) that the
// FP8 dot kernel applies to weights and activations, for every pair of bytes
// in both halves of a word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"

using namespace nvfp4;

// word i holds the 8 codes of the fp32 bit patterns (first + 8 i + j) | sign,
// j = 0..7, code j in bits 4 j .. 4 j + 3
__global__ void e2m1_sweep_kernel(uint32_t first, uint32_t sign, int64_t nwords, uint32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const uint32_t b = first + 8u * (uint32_t)i;
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = __uint_as_float((b + (uint32_t)j) | sign);
  uint32_t c = 0u;
  c = NVFP4_CVT_PK_FP4(c, q[0], q[1], 0);
  c = NVFP4_CVT_PK_FP4(c, q[2], q[3], 1);
  c = NVFP4_CVT_PK_FP4(c, q[4], q[5], 2);
  c = NVFP4_CVT_PK_FP4(c, q[6], q[7], 3);
  out[i] = fix_zero_signs(c);
}

// One workgroup per E4M3 scale byte (0..126), one thread per code byte
// (0..255, low nibble first).  Row (scale, byte) of each output holds the
// pair of 16-bit results for the byte's two codes:
//   f32route: bf16 bits of code * s (dequant8)
//   f16route: f16 bits of code * s (split_scale + dequant8_f16)
//   f16s:     f16 bits of code * s (the scale itself as the converter's scale,
//             scale_mantissa_f16 + dequant8_f16)
//   pow2bf16: bf16 bits of code * e2, e2 = 2^e of s (v_cvt_scalef32_pk_bf16_fp4)
// and per scale byte e2 (fp32) and mu (f16 bits) of split_scale.
__global__ void dequant_table_kernel(uint32_t* __restrict__ f32route, uint32_t* __restrict__ f16route,
                                     uint32_t* __restrict__ f16s, uint32_t* __restrict__ pow2bf16,
                                     float* __restrict__ e2_out, uint16_t* __restrict__ mu_out) {
  const uint32_t sbyte = blockIdx.x, cbyte = threadIdx.x;
  const float s = NVFP4_E4M3_TO_F32(sbyte, 0);
  float e2;
  f16x2 mu;
  split_scale(s, &e2, &mu);
  // the code byte in position 0 of a word whose other bytes differ, so that
  // a wrong byte select would show
  const uint32_t w = cbyte | ((cbyte ^ 0x5Au) << 8) | ((cbyte ^ 0xA5u) << 16) | ((cbyte ^ 0xFFu) << 24);
  const bf16x8 a = dequant8(w, s);
  const f16x8 h = dequant8_f16(w, e2, mu);
  const f16x8 hs = dequant8_f16(w, s, scale_mantissa_f16(s));
  const bf16x2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, e2, 0);
  const int o = (int)(sbyte * 256 + cbyte);
  f32route[o] = __builtin_bit_cast(u32x4, a)[0];
  const f16x2 h01 = {h[0], h[1]};
  f16route[o] = __builtin_bit_cast(uint32_t, h01);
  const f16x2 hs01 = {hs[0], hs[1]};
  f16s[o] = __builtin_bit_cast(uint32_t, hs01);
  pow2bf16[o] = __builtin_bit_cast(uint32_t, p);
  if (cbyte == 0) {
    e2_out[sbyte] = e2;
    mu_out[sbyte] = __builtin_bit_cast(uint16_t, mu[0]);
  }
}

// thread t (0..65535): the byte pair (t & 0xFF, t >> 8) in the low half of a
// word (lo) and in the high half (hi), the other half holding different bytes
__global__ void e4m3_bf16_table_kernel(uint32_t* __restrict__ lo, uint32_t* __restrict__ hi) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  lo[t] = __builtin_bit_cast(uint32_t, NVFP4_E4M3X2_TO_BF16(t | ((t ^ 0x5A5Au) << 16), false));
  hi[t] = __builtin_bit_cast(uint32_t, NVFP4_E4M3X2_TO_BF16((t << 16) | (t ^ 0xA5A5u), true));
}

extern "C" {

// count values starting at bit pattern first (count % 8 == 0, count > 0,
// first + count <= 2^31); sign_bit 0 or 0x80000000; out: count / 8 words.
// Returns 0, or -1 for arguments outside those rules, or the HIP error.
int nvfp4_test_e2m1_sweep(uint32_t first, uint32_t sign_bit, int64_t count, uint32_t* out, void* stream) {
  if (out == nullptr || count <= 0 || count % 8 != 0 || (int64_t)first + count > ((int64_t)1 << 31) ||
      (sign_bit != 0u && sign_bit != 0x80000000u))
    return -1;
  const int64_t nwords = count / 8;
  const int threads = 256;
  hipLaunchKernelGGL(e2m1_sweep_kernel, dim3((unsigned)((nwords + threads - 1) / threads)), dim3(threads), 0,
                     (hipStream_t)stream, first, sign_bit, nwords, out);
  return (int)hipGetLastError();
}

// outputs sized 127 * 256 (words) and 127 (e2, mu)
int nvfp4_test_dequant_table(uint32_t* f32route, uint32_t* f16route, uint32_t* f16s, uint32_t* pow2bf16, float* e2,
                             uint16_t* mu, void* stream) {
  if (!f32route || !f16route || !f16s || !pow2bf16 || !e2 || !mu) return -1;
  hipLaunchKernelGGL(dequant_table_kernel, dim3(127), dim3(256), 0, (hipStream_t)stream, f32route, f16route, f16s,
                     pow2bf16, e2, mu);
  return (int)hipGetLastError();
}

// outputs sized 65536 words each
int nvfp4_test_e4m3_bf16_table(uint32_t* lo, uint32_t* hi, void* stream) {
  if (!lo || !hi) return -1;
  hipLaunchKernelGGL(e4m3_bf16_table_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, lo, hi);
  return (int)hipGetLastError();
}

}  // extern "C"
