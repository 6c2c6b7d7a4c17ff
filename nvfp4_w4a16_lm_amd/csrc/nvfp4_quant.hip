// Online NVFP4 quantization kernels for gfx950.
//
// Method: vLLM API docs, quantization.online.lm_head, _quantize_nvfp4 --
// a tensor-wide amax gives the fp32 global scale amax / (6 * 448) (clamped at
// 1e-12); every 16 consecutive weights of a row share an E4M3 block scale;
// weights are rounded to the E2M1 grid with a sign bit and packed two per
// byte, low nibble first.
//
// Launch sequence on one stream (no host sync, no allocation, no memset node):
//   1. amax_init     : global_scale word <- 0 (it accumulates |amax| bits)
//   2. amax          : one integer atomic max per workgroup
//   3. global_scale  : 1 thread turns the amax bits into the fp32 global scale
//   4. quant_pack    : every thread re-derives 1/gs and encodes 16-weight blocks
//
// The weight, packed codes and scales are viewed as flat arrays: with
// K % 16 == 0 each 16-block lies inside one row and block b covers weights
// [16b, 16b+16), packed bytes [8b, 8b+8) and scale byte b.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr int kThreads = 256;

__global__ void amax_init_kernel(uint32_t* __restrict__ amax_bits) {
  if (threadIdx.x == 0) *amax_bits = 0u;
}

// Tensor-wide max |w|: bf16 magnitudes compared as unsigned 16-bit integers
// (order-preserving for finite values), 4 x 16-byte loads in flight per
// thread, then a wavefront butterfly and one atomic per workgroup.  The word
// receives the magnitude as fp32 bits, which order like unsigned integers.
__global__ __launch_bounds__(kThreads) void amax_kernel(const u32x4* __restrict__ w, int64_t n16,
                                                        uint32_t* __restrict__ amax_bits) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m0 = 0, m1 = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = load_stream16(w + i);
    const u32x4 b = load_stream16(w + i + stride);
    const u32x4 c = load_stream16(w + i + 2 * stride);
    const u32x4 d = load_stream16(w + i + 3 * stride);
    m0 = pk_max_u16(m0, a.x & 0x7FFF7FFFu); m1 = pk_max_u16(m1, a.y & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, a.z & 0x7FFF7FFFu); m1 = pk_max_u16(m1, a.w & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, b.x & 0x7FFF7FFFu); m1 = pk_max_u16(m1, b.y & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, b.z & 0x7FFF7FFFu); m1 = pk_max_u16(m1, b.w & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, c.x & 0x7FFF7FFFu); m1 = pk_max_u16(m1, c.y & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, c.z & 0x7FFF7FFFu); m1 = pk_max_u16(m1, c.w & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, d.x & 0x7FFF7FFFu); m1 = pk_max_u16(m1, d.y & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, d.z & 0x7FFF7FFFu); m1 = pk_max_u16(m1, d.w & 0x7FFF7FFFu);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = load_stream16(w + i);
    m0 = pk_max_u16(m0, a.x & 0x7FFF7FFFu); m1 = pk_max_u16(m1, a.y & 0x7FFF7FFFu);
    m0 = pk_max_u16(m0, a.z & 0x7FFF7FFFu); m1 = pk_max_u16(m1, a.w & 0x7FFF7FFFu);
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
    atomicMax(amax_bits, v << 16);
  }
}

// gs = max(fl32(amax / 2688), fl32(1e-12)); IEEE division (no fast-math).
__global__ void global_scale_kernel(float* __restrict__ gs_word) {
  if (threadIdx.x == 0) {
    const float a = __uint_as_float(*reinterpret_cast<const uint32_t*>(gs_word));
    const float gs = a / (kE2m1Max * kE4m3Max);
    *gs_word = fmaxf(gs, 1e-12f);
  }
}

// Encode one 16-weight block held in eight 32-bit words (weight i in the low
// half of d[i/2] when i is even).  Writes 8 packed bytes and the scale byte.
__device__ __forceinline__ void encode_block(const uint32_t d[8], float inv, uint2* out_codes,
                                             uint32_t* out_scale) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = pk_max_u16(m, d[i] & 0x7FFF7FFFu);
  const float bmax = __uint_as_float(max(m & 0xFFFFu, m >> 16) << 16);
  const float t = bmax / kE2m1Max;       // fl32(b / 6)
  const float u = fminf(t * inv, kE4m3Max);
  float s;
  const uint32_t sbyte = e4m3_encode_rne(u, &s);
  const float r = (s > 0.0f) ? inv / s : 0.0f;   // fl32(inv / s); zero block -> codes 0
  float q[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[2 * i] = bf16_lo(d[i]) * r;       // fl32(w * r)
    q[2 * i + 1] = bf16_hi(d[i]) * r;
  }
  uint32_t lo = 0u, hi = 0u;
  lo = NVFP4_CVT_PK_FP4(lo, q[0], q[1], 0);
  lo = NVFP4_CVT_PK_FP4(lo, q[2], q[3], 1);
  lo = NVFP4_CVT_PK_FP4(lo, q[4], q[5], 2);
  lo = NVFP4_CVT_PK_FP4(lo, q[6], q[7], 3);
  hi = NVFP4_CVT_PK_FP4(hi, q[8], q[9], 0);
  hi = NVFP4_CVT_PK_FP4(hi, q[10], q[11], 1);
  hi = NVFP4_CVT_PK_FP4(hi, q[12], q[13], 2);
  hi = NVFP4_CVT_PK_FP4(hi, q[14], q[15], 3);
  *out_codes = make_uint2(fix_zero_signs(lo), fix_zero_signs(hi));
  *out_scale = sbyte;
}

// One thread per 16-weight block: two 16-byte loads, one 8-byte store of codes
// and one scale byte.  Consecutive threads own consecutive blocks, so a
// wavefront reads 2 KiB and writes 512 + 64 contiguous bytes.
__global__ __launch_bounds__(kThreads) void quant_pack_kernel(const u32x4* __restrict__ w, int64_t nblocks,
                                                              const float* __restrict__ gs_ptr,
                                                              uint2* __restrict__ packed,
                                                              uint8_t* __restrict__ scales) {
  const float inv = 1.0f / *gs_ptr;     // fl32(1 / gs), IEEE division
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    const u32x4 lo = load_stream16(w + 2 * b);
    const u32x4 hi = load_stream16(w + 2 * b + 1);
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint2 codes;
    uint32_t sb;
    encode_block(d, inv, &codes, &sb);
    packed[b] = codes;
    scales[b] = (uint8_t)sb;
  }
}

static int grid_for(int64_t work_items, int per_thread, int max_blocks) {
  const int64_t threads = (work_items + per_thread - 1) / per_thread;
  int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > max_blocks) blocks = max_blocks;
  return (int)blocks;
}

hipError_t launch_quantize(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                           float* global_scale, hipStream_t stream) {
  const int64_t n16 = N * K / 8;        // 16-byte words of the weight
  const int64_t nblocks = N * K / kGroup;
  uint32_t* bits = reinterpret_cast<uint32_t*>(global_scale);
  hipError_t e;
  e = launch_kernel((const void*)amax_init_kernel, dim3(1), dim3(64), stream, bits);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)amax_kernel, dim3(grid_for(n16, 4, 256 * 32)), dim3(kThreads), stream,
                    reinterpret_cast<const u32x4*>(W), n16, bits);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)global_scale_kernel, dim3(1), dim3(64), stream, global_scale);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)quant_pack_kernel, dim3(grid_for(nblocks, 1, 256 * 64)), dim3(kThreads),
                    stream, reinterpret_cast<const u32x4*>(W), nblocks, (const float*)global_scale,
                    reinterpret_cast<uint2*>(packed), scales);
  return e;
}

}  // namespace nvfp4
