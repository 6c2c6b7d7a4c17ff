// Online NVFP4 quantization kernels for gfx950.
//
// Method: vLLM API docs, quantization.online.lm_head, _quantize_nvfp4 --
// a tensor-wide amax gives the fp32 global scale amax / (6 * 448) (clamped at
// 1e-12); every 16 consecutive weights of a row share an E4M3 block scale;
// weights are rounded to the E2M1 grid with a sign bit and packed two per
// byte, low nibble first.
//
// Launch sequence on one stream (no host sync, no allocation, no memset node):
//   1. amax_init  : global_scale word <- 0x80000000 (a tagged amax of 0)
//   2. amax       : integer atomic max of (0x80000000 | |w|max as fp32 bits),
//                   one per workgroup
//   3. quant_pack : every workgroup reads the word: tagged -> the amax, from
//                   which it derives gs = max(amax/2688, 1e-12); untagged ->
//                   gs itself.  Workgroup 0 stores the untagged gs.  Both
//                   forms give the same gs, so the order of that store
//                   against the other workgroups' reads does not matter.
//
// Memory access: HBM streams fastest when each workgroup walks a contiguous
// span with every wavefront instruction covering 1 KiB (measured ~7 TB/s on
// MI355X, against ~6 TB/s for grid-stride loops), so both streaming kernels
// split the weight into one contiguous span per workgroup (amax: ~1024 long
// spans; quant_pack: 64 KiB spans).
// quant_pack walks the tensor from its end, so its first reads find the tail
// of the weight that amax read last; it collects each 64 KiB span's codes and
// scales in LDS and writes them in one burst at the end of the span.
//
// The weight, packed codes and scales are viewed as flat arrays: with
// K % 16 == 0 each 16-block lies inside one row; 16-byte vector v holds
// weights [8v, 8v+8), i.e. half of block v/2, whose codes are packed
// 32-bit word v and whose scale is byte v/2.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                  // 16-byte vectors in flight per thread
constexpr int kSpan = 4096;                 // 16-byte vectors per quant_pack span (64 KiB of weights)
constexpr uint32_t kTag = 0x80000000u;      // marks the word as holding an amax

__global__ void amax_init_kernel(uint32_t* __restrict__ word) {
  if (threadIdx.x == 0) *word = kTag;
}

// Tensor-wide max |w| over workgroup span [b0, b1) of 16-byte vectors:
// bf16 magnitudes compared as unsigned 16-bit integers (order-preserving for
// finite values), a wavefront butterfly, then one atomic per workgroup.
__global__ __launch_bounds__(kThreads) void amax_kernel(const u32x4* __restrict__ w, int64_t n16, int64_t per_wg,
                                                        uint32_t* __restrict__ word) {
  const int64_t b0 = (int64_t)blockIdx.x * per_wg;
  const int64_t b1 = min(n16, b0 + per_wg);
  uint32_t m0 = 0, m1 = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += kThreads * kUnroll) {
    u32x4 v[kUnroll];
    // clamped, unconditional loads (a branch around a load makes the compiler
    // wait for it); a repeated vector cannot change the max
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_stream16(w + min(i + kThreads * u, b1 - 1));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      m0 = pk_max_u16(m0, v[u].x & 0x7FFF7FFFu);
      m1 = pk_max_u16(m1, v[u].y & 0x7FFF7FFFu);
      m0 = pk_max_u16(m0, v[u].z & 0x7FFF7FFFu);
      m1 = pk_max_u16(m1, v[u].w & 0x7FFF7FFFu);
    }
  }
  m0 = pk_max_u16(m0, m1);
  uint32_t r = max(m0 & 0xFFFFu, m0 >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) r = max(r, (uint32_t)__shfl_xor((int)r, off, 64));
  __shared__ uint32_t part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = part[0];
#pragma unroll
    for (int j = 1; j < kThreads / 64; ++j) v = max(v, part[j]);
    atomicMax(word, kTag | (v << 16));
  }
}

// fl32(b / 6) for b >= 0 from a multiply and two fused multiply-adds:
// q0 = fl(b * fl(1/6)); the residual b - 6 q0 is exact in fp32, and one
// correction step gives the correctly rounded quotient for every finite
// bf16 b (checked exhaustively against exact rational arithmetic on the host).
__device__ __forceinline__ float div6(float b) {
  const float inv6 = 0.16666667163372039795f;    // fl32(1/6)
  const float q0 = b * inv6;
  const float r = __builtin_fmaf(-q0, 6.0f, b);
  return __builtin_fmaf(r, inv6, q0);
}

// Encode the 8 weights of one 16-byte vector (half a block).  The other half
// of the block is in the neighbouring lane (lane ^ 1), which supplies its
// half-block max through a DPP quad swap.  Returns the packed codes; *sbyte
// receives the block's E4M3 scale byte.
__device__ __forceinline__ uint32_t encode_half_block(const u32x4 v, float inv, const float* __restrict__ rlut,
                                                      uint32_t* sbyte) {
  const uint32_t m = pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
  uint32_t mh = max(m & 0xFFFFu, m >> 16);
  mh = max(mh, (uint32_t)__builtin_amdgcn_mov_dpp((int)mh, 0xB1, 0xF, 0xF, true));   // lane ^ 1
  const float bmax = __uint_as_float(mh << 16);
  const float t = div6(bmax);                      // fl32(b / 6)
  const float u = fminf(t * inv, kE4m3Max);        // fl32(t * inv), clamped to 448
  float s;
  const uint32_t sb = e4m3_encode_rne(u, &s);
  const float r = rlut[sb];                        // fl32(inv / s), 0 when s == 0
  const float q0 = bf16_lo(v.x) * r, q1 = bf16_hi(v.x) * r;
  const float q2 = bf16_lo(v.y) * r, q3 = bf16_hi(v.y) * r;
  const float q4 = bf16_lo(v.z) * r, q5 = bf16_hi(v.z) * r;
  const float q6 = bf16_lo(v.w) * r, q7 = bf16_hi(v.w) * r;
  uint32_t c = 0u;
  c = NVFP4_CVT_PK_FP4(c, q0, q1, 0);
  c = NVFP4_CVT_PK_FP4(c, q2, q3, 1);
  c = NVFP4_CVT_PK_FP4(c, q4, q5, 2);
  c = NVFP4_CVT_PK_FP4(c, q6, q7, 3);
  *sbyte = sb;
  return fix_zero_signs(c);
}

// One kSpan-vector span per workgroup, taken from the end of the tensor
// (workgroup 0 gets the last span).
// gs_word: the tagged amax or the global scale itself; gs_out (may be null):
// where workgroup 0 stores the global scale.
__global__ __launch_bounds__(kThreads) void quant_pack_kernel(const u32x4* __restrict__ w, int64_t n16,
                                                              const float* gs_word, float* gs_out,
                                                              uint32_t* __restrict__ packed,
                                                              uint8_t* __restrict__ scales) {
  __shared__ float rlut[128];
  // the span's codes and scale bytes, written out in one burst at the end
  __shared__ __attribute__((aligned(16))) uint32_t code_stage[kSpan];
  __shared__ __attribute__((aligned(16))) uint32_t scale_stage[kSpan / 8];
  const uint32_t word = *reinterpret_cast<const uint32_t*>(gs_word);
  float gs;
  if (word & kTag) {
    const float a = __uint_as_float(word & ~kTag);
    gs = fmaxf(a / (kE2m1Max * kE4m3Max), 1e-12f);   // IEEE division
  } else {
    gs = __uint_as_float(word);
  }
  if (gs_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  const float inv = 1.0f / gs;                        // fl32(1 / gs)
  if (threadIdx.x < 128) {
    // r for E4M3 byte threadIdx.x (0..126 are the finite non-negative scales)
    const float s = NVFP4_E4M3_TO_F32(threadIdx.x, 0);
    rlut[threadIdx.x] = (threadIdx.x != 0x7F && s > 0.0f) ? inv / s : 0.0f;
  }
  __syncthreads();

  const int64_t span = (int64_t)(gridDim.x - 1 - blockIdx.x);
  const int64_t b0 = span * kSpan;
  const int64_t b1 = min(n16, b0 + kSpan);
  for (int64_t i = b0 + threadIdx.x; i < b1; i += kThreads * kUnroll) {
    u32x4 v[kUnroll];
    // clamped, unconditional loads; vectors past the span end are encoded
    // (from a repeated vector) but never stored
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_stream16(w + min(i + kThreads * u, b1 - 1));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t vi = i + kThreads * u;
      uint32_t sb;
      const uint32_t codes = encode_half_block(v[u], inv, rlut, &sb);
      if (vi < b1) {
        code_stage[vi - b0] = codes;
        if ((vi & 1) == 0) reinterpret_cast<uint8_t*>(scale_stage)[(vi - b0) >> 1] = (uint8_t)sb;
      }
    }
  }
  // Burst out the span: interleaving small code and scale stores with the
  // weight stream costs far more HBM time than writing each span's 16 KiB of
  // codes and 2 KiB of scales contiguously at its end (measured on MI355X).
  __syncthreads();
  const int nc = (int)(b1 - b0);                       // code words (even: b0, n16 even)
  uint32_t* const pd = packed + b0;
  for (int i = 4 * (int)threadIdx.x; i < nc; i += 4 * kThreads) {
    if (i + 4 <= nc)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&code_stage[i]), reinterpret_cast<u32x4*>(pd + i));
    else
      for (int e = i; e < nc; ++e) __builtin_nontemporal_store(code_stage[e], pd + e);
  }
  const int ns = nc >> 1;                              // scale bytes; the destination is 4-byte aligned
  uint8_t* const sd = scales + (b0 >> 1);
  for (int i = 4 * (int)threadIdx.x; i < ns; i += 4 * kThreads) {
    if (i + 4 <= ns) {
      __builtin_nontemporal_store(scale_stage[i >> 2], reinterpret_cast<uint32_t*>(sd + i));
    } else {
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(scale_stage);
      for (int e = i; e < ns; ++e) sd[e] = sb[e];
    }
  }
}

hipError_t launch_quantize(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                           float* global_scale, hipStream_t stream) {
  const int64_t n16 = N * K / 8;                 // 16-byte vectors of the weight (even: K % 16 == 0)
  uint32_t* word = reinterpret_cast<uint32_t*>(global_scale);
  // amax: about 1024 workgroups, each one contiguous span of a multiple of
  // 512 vectors (long spans stream best: 1024 spans beat 4096 by ~11 %).
  // quant_pack: one span of kSpan vectors per workgroup, whose codes and
  // scales fit its LDS staging.  Both span sizes are multiples of 512, so a
  // block never straddles two workgroups and lane parity equals vector parity
  // in every iteration (the two halves of a block sit in lanes 2j, 2j+1).
  const int64_t amax_span = std::max<int64_t>(512, ((n16 + 1023) / 1024 + 511) / 512 * 512);
  const int amax_grid = (int)((n16 + amax_span - 1) / amax_span);
  const int pack_grid = (int)((n16 + kSpan - 1) / kSpan);
  hipError_t e;
  e = launch_kernel((const void*)amax_init_kernel, dim3(1), dim3(64), stream, word);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)amax_kernel, dim3(amax_grid), dim3(kThreads), stream,
                    reinterpret_cast<const u32x4*>(W), n16, amax_span, word);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)quant_pack_kernel, dim3(pack_grid), dim3(kThreads), stream,
                    reinterpret_cast<const u32x4*>(W), n16, (const float*)global_scale, global_scale,
                    reinterpret_cast<uint32_t*>(packed), scales);
  return e;
}

// Activations of a W4A4 layer: the same block scales and codes with a given
// (static) global scale; no amax pass, nothing written back to it.
hipError_t launch_quantize_given_scale(const void* X, int64_t M, int64_t K, const float* global_scale,
                                       uint8_t* packed, uint8_t* scales, hipStream_t stream) {
  const int64_t n16 = M * K / 8;
  const int pack_grid = (int)((n16 + kSpan - 1) / kSpan);
  return launch_kernel((const void*)quant_pack_kernel, dim3(pack_grid), dim3(kThreads), stream,
                       reinterpret_cast<const u32x4*>(X), n16, global_scale, (float*)nullptr,
                       reinterpret_cast<uint32_t*>(packed), scales);
}

}  // namespace nvfp4
