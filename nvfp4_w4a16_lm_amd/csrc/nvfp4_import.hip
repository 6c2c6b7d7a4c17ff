// Adopting a pre-quantized NVFP4 checkpoint for the W4A16 GEMM.
//
// Method: vLLM modelopt.py, class KNvfp4Static (create_weights fills the
// block scales with NaN so that an unloaded scale is detectable; process
// rejects a scale that is still NaN, warns when the partitions'
// weight_scale_2 values differ, and keeps their maximum as the
// dequantization-direction global scale); vLLM API docs,
// compressed_tensors.schemes, class CompressedTensorsW4A16Fp4
// (weight_global_scale is stored inverted; the global scale is 1 / its
// maximum, one float32 division).  The packed codes and block scales keep the
// layout nvfp4_w4a16_gemm reads, so nothing else changes.
//
// import_prepare_kernel (one wavefront): collapses the P partition scales
//   into the global scale and writes the flags word with the partition and
//   global-scale bits (the not-loaded bit starts clear).
// scale_nan_scan_kernel: streams the block scales once, 16-byte loads, four
//   per thread, one contiguous 16 KiB span per workgroup; a wavefront that saw
//   an e4m3fn NaN byte (0x7F or 0xFF) ORs the not-loaded bit into the flags
//   word with one atomic.
// fill_sentinel_kernel: writes 0x7F into every block-scale byte.
#include <algorithm>
#include <climits>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr uint32_t kFlagScalesNotLoaded = 1u;
constexpr uint32_t kFlagPartitionsDiffer = 2u;
constexpr uint32_t kFlagBadGlobalScale = 4u;
constexpr uint32_t kCanonicalNaN = 0x7FC00000u;
constexpr int kScanThreads = 256;
constexpr int kScanVecsPerThread = 4;
constexpr int kScanSpan = kScanThreads * kScanVecsPerThread;   // 16-byte vectors per workgroup

// (value, index) with NaN sticking and, on equal values (+0 / -0), the lower
// index winning: the first partition's value is kept on ties, as a
// left-to-right maximum keeps it.
struct MaxPick {
  float v;
  int i;
  bool nan;
};

__device__ __forceinline__ MaxPick max_pick(MaxPick a, MaxPick b) {
  if (a.nan || b.nan) return MaxPick{0.f, 0, true};
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__global__ __launch_bounds__(64) void import_prepare_kernel(const float* __restrict__ part, int P, int convention,
                                                            float* __restrict__ gs_out,
                                                            uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x;
  const float first = part[0];
  MaxPick best{-__builtin_huge_valf(), INT_MAX, false};   // loses to every element
  bool differ = false;
  for (int p = lane; p < P; p += 64) {
    const float v = part[p];
    best = max_pick(best, MaxPick{v, p, v != v});
    differ |= p > 0 && !(v == first);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const MaxPick o{__shfl_xor(best.v, off, 64), __shfl_xor(best.i, off, 64), (bool)__shfl_xor((int)best.nan, off, 64)};
    best = max_pick(best, o);
  }
  differ = __ballot(differ) != 0;
  if (lane == 0) {
    float m = best.nan ? __uint_as_float(kCanonicalNaN) : best.v;
    float gs = convention == 0 ? m : 1.0f / m;   // IEEE division (compressed-tensors stores the inverse)
    if (gs != gs) gs = __uint_as_float(kCanonicalNaN);
    uint32_t f = 0;
    if (differ) f |= kFlagPartitionsDiffer;
    if (!(gs > 0.f && gs <= 3.40282347e38f)) f |= kFlagBadGlobalScale;
    *gs_out = gs;
    *flags = f;
  }
}

// Nonzero iff some byte of w is 0x7F or 0xFF: clearing bit 7 leaves bytes <=
// 0x7F, and adding 1 to each carries into bit 7 only from 0x7F (no carry can
// cross into the next byte).
__device__ __forceinline__ uint32_t nan_bytes(uint32_t w) {
  return ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

__global__ __launch_bounds__(kScanThreads) void scale_nan_scan_kernel(const uint8_t* __restrict__ scales,
                                                                      int64_t nbytes,
                                                                      uint32_t* __restrict__ flags) {
  const int64_t nvec = nbytes >> 4;
  const u32x4* vec = reinterpret_cast<const u32x4*>(scales);
  const int64_t base = (int64_t)blockIdx.x * kScanSpan + threadIdx.x;
  uint32_t seen = 0;
  if (nvec > 0) {
    u32x4 v[kScanVecsPerThread];
#pragma unroll
    for (int j = 0; j < kScanVecsPerThread; ++j)
      v[j] = vec[min(base + (int64_t)j * kScanThreads, nvec - 1)];   // clamped: re-reads the last vector
#pragma unroll
    for (int j = 0; j < kScanVecsPerThread; ++j)
      seen |= nan_bytes(v[j].x) | nan_bytes(v[j].y) | nan_bytes(v[j].z) | nan_bytes(v[j].w);
  }
  // the bytes after the last whole vector: the last workgroup's first threads
  const int64_t tail = nbytes - (nvec << 4);
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < tail) {
    const uint32_t b = scales[(nvec << 4) + threadIdx.x];
    seen |= nan_bytes(b);
  }
  if (__ballot(seen != 0) != 0 && (threadIdx.x & 63) == 0) atomicOr(flags, kFlagScalesNotLoaded);
}

__global__ __launch_bounds__(kScanThreads) void fill_sentinel_kernel(uint8_t* __restrict__ scales, int64_t nbytes) {
  const int64_t nvec = nbytes >> 4;
  u32x4* vec = reinterpret_cast<u32x4*>(scales);
  const int64_t base = (int64_t)blockIdx.x * kScanSpan + threadIdx.x;
  const u32x4 s{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
#pragma unroll
  for (int j = 0; j < kScanVecsPerThread; ++j) {
    const int64_t i = base + (int64_t)j * kScanThreads;
    if (i < nvec) vec[i] = s;
  }
  const int64_t tail = nbytes - (nvec << 4);
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < tail) scales[(nvec << 4) + threadIdx.x] = 0x7F;
}

static unsigned scan_grid(int64_t nbytes) {
  const int64_t nvec = nbytes >> 4;
  return (unsigned)std::max<int64_t>(1, (nvec + kScanSpan - 1) / kScanSpan);
}

hipError_t launch_import(const float* partition_scales, int64_t P, int convention, const uint8_t* scales,
                         int64_t nbytes, float* global_scale, uint32_t* flags, hipStream_t stream) {
  hipError_t e = launch_kernel((const void*)import_prepare_kernel, dim3(1), dim3(64), stream, partition_scales,
                               (int)P, convention, global_scale, flags);
  if (e != hipSuccess) return e;
  return launch_kernel((const void*)scale_nan_scan_kernel, dim3(scan_grid(nbytes)), dim3(kScanThreads), stream,
                       scales, nbytes, flags);
}

hipError_t launch_fill_sentinel(uint8_t* scales, int64_t nbytes, hipStream_t stream) {
  return launch_kernel((const void*)fill_sentinel_kernel, dim3(scan_grid(nbytes)), dim3(kScanThreads), stream,
                       scales, nbytes);
}

}  // namespace nvfp4
