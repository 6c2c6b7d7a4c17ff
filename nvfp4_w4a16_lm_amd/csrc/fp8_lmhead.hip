// The FP8 lm_head copy: per-row E4M3 weight scales, per-token dynamic E4M3
// activation scales, and the scaled FP8 GEMM that computes logits from them.
//
// Method: vLLM API docs, quantization.online.lm_head, quantized_lm_head_copy
// (the "fp8" copy: per-row weight and per-token activation scales on an FP8
// linear kernel); vLLM modelopt.py, KFp8StaticChannel (float8_e4m3fn weight
// [N, K], one float32 scale per output row) and the FP8_PER_CHANNEL_PER_TOKEN
// recipe; vLLM API docs, compressed_tensors.schemes, the W8A8 FP8
// apply_weights path (per-token quantization of the input, then a scaled
// matmul with the token scales, the row scales, the input dtype as output
// dtype and the bias).
//
// Row rule (weights per output row, activations per token), the plainest
// reading of the pages: s = max(amax / 448, 1e-12) in float32, q =
// e4m3(clamp(x * (1 / s), -448, 448)), round to nearest even, sign kept.
//
// fp8_quant_rows_kernel<V>: one wavefront per row; the row's largest |x|
//   (bf16 magnitudes compare as integers), a wavefront butterfly, then 8
//   values per lane converted with v_cvt_pk_fp8_f32; rows up to 8192 values
//   stay in registers between the two steps (read from HBM once).
// fp8_gemm_kernel<MT>: a workgroup of 4 wavefronts owns 128 weight rows and
//   16 MT activation rows (MT <= 8); K is walked in 64-byte slabs staged in
//   double-buffered LDS (next slab's global loads in registers while the
//   current one computes).  Each wavefront computes 32 rows x 16 MT with
//   v_mfma_f32_16x16x32_fp8_fp8.  Within a slab, lane (r, g) = (l % 16,
//   l / 16) reads the 16 contiguous bytes [16 g, 16 g + 16) of its row, and
//   MFMA step j uses bytes 8 j .. 8 j + 7 of them: the k order inside the
//   slab is permuted identically for both operands, which leaves the sum
//   unchanged.  LDS rows are 64 bytes, 16-byte piece p of row r at slot
//   p ^ ((r >> 2) & 3), so 8 consecutive lanes read 8 different bank groups.
//   Pieces past K are zero in both operands.  Epilogue: acc * s_x[m] *
//   s_w[n] (+ bias[n]) in float32, one rounding to bf16.
#include <algorithm>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

constexpr float kFp8Max = 448.0f;
constexpr float kFp8ScaleMin = 1e-12f;

// Largest bf16 magnitude (as its bit pattern) of the 8 values of a vector.
__device__ __forceinline__ uint32_t mag_max8(const u32x4 d) {
  const uint32_t a = max(max(d.x & 0x7FFFu, (d.x >> 16) & 0x7FFFu), max(d.y & 0x7FFFu, (d.y >> 16) & 0x7FFFu));
  const uint32_t b = max(max(d.z & 0x7FFFu, (d.z >> 16) & 0x7FFFu), max(d.w & 0x7FFFu, (d.w >> 16) & 0x7FFFu));
  return max(a, b);
}

// 8 bf16 values times inv, clamped to +-448, as 8 e4m3 bytes (RNE).
__device__ __forceinline__ uint2 to_e4m3x8(const u32x4 d, float inv) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = fminf(fmaxf(bf16_lo(d[e]) * inv, -kFp8Max), kFp8Max);
    f[2 * e + 1] = fminf(fmaxf(bf16_hi(d[e]) * inv, -kFp8Max), kFp8Max);
  }
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2(lo, hi);
}

// V > 0: the lane's V vectors of the row stay in registers between the two
// passes (K <= 512 V), so the row is read once; V == 0: any K, the row is
// read a second time for the conversion.
template <int V>
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t* __restrict__ a, int64_t R, int K,
                                                             uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int nvec = K >> 3;                                       // 8 bf16 per 16-byte vector
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < R; row += (int64_t)gridDim.x * 4) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a + row * K);
    uint2* dst = reinterpret_cast<uint2*>(q + row * K);
    u32x4 buf[V > 0 ? V : 1];
    uint32_t mx = 0;
    if constexpr (V > 0) {
      // clamped, unconditional loads; a repeated vector does not change the max
#pragma unroll
      for (int j = 0; j < V; ++j) buf[j] = src[min(lane + 64 * j, nvec - 1)];
#pragma unroll
      for (int j = 0; j < V; ++j) mx = max(mx, mag_max8(buf[j]));
    } else {
      for (int v = lane; v < nvec; v += 64) mx = max(mx, mag_max8(src[v]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    const float amax = __uint_as_float(mx << 16);
    const float s = fmaxf(amax / kFp8Max, kFp8ScaleMin);          // IEEE division
    const float inv = 1.0f / s;
    if (lane == 0) scales[row] = s;
    if constexpr (V > 0) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (lane + 64 * j < nvec) dst[lane + 64 * j] = to_e4m3x8(buf[j], inv);
    } else {
      for (int v = lane; v < nvec; v += 64) dst[v] = to_e4m3x8(src[v], inv);
    }
  }
}

constexpr int kFp8Rows = 128;     // weight rows per workgroup
constexpr int kFp8Slab = 64;      // k bytes per LDS slab

template <int MT>
__global__ __launch_bounds__(256) void fp8_gemm_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                       int M, int K, const uint8_t* __restrict__ wq,
                                                       const float* __restrict__ ws, int N,
                                                       const uint16_t* __restrict__ bias,
                                                       uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MT;
  constexpr int kWPieces = kFp8Rows * 4 / 256;                  // 16-byte W pieces per thread per slab
  constexpr int kXPieces = (BM * 4 + 255) / 256;                // 16-byte X pieces per thread per slab
  __shared__ __attribute__((aligned(16))) uint8_t wl[2][kFp8Rows * kFp8Slab];
  __shared__ __attribute__((aligned(16))) uint8_t xl[2][BM * kFp8Slab];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kFp8Rows, m0 = blockIdx.y * BM;
  const int nslabs = (K + kFp8Slab - 1) / kFp8Slab;

  // piece i of the slab: row i >> 2, piece i & 3, stored at slot (i & 3) ^ ((row >> 2) & 3)
  auto slot_of = [](int row, int p) { return row * kFp8Slab + 16 * (p ^ ((row >> 2) & 3)); };
  u32x4 wreg[kWPieces], xreg[kXPieces];
  auto load = [&](int sb) {
    const int kb = sb * kFp8Slab;
#pragma unroll
    for (int j = 0; j < kWPieces; ++j) {
      const int i = tid + 256 * j, row = i >> 2, p = i & 3;
      const int64_t n = min(n0 + row, N - 1);
      const int k = kb + 16 * p;
      const u32x4 v = *reinterpret_cast<const u32x4*>(wq + n * K + min(k, K - 16));
      wreg[j] = k < K ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kXPieces; ++j) {
      const int i = tid + 256 * j, row = i >> 2, p = i & 3;
      const int64_t m = min(m0 + min(row, BM - 1), M - 1);
      const int k = kb + 16 * p;
      const u32x4 v = *reinterpret_cast<const u32x4*>(xq + m * K + min(k, K - 16));
      xreg[j] = (k < K && i < BM * 4) ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int j = 0; j < kWPieces; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<u32x4*>(&wl[b][slot_of(i >> 2, i & 3)]) = wreg[j];
    }
#pragma unroll
    for (int j = 0; j < kXPieces; ++j) {
      const int i = tid + 256 * j;
      if (i < BM * 4) *reinterpret_cast<u32x4*>(&xl[b][slot_of(i >> 2, i & 3)]) = xreg[j];
    }
  };

  f32x4 acc[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int sb = 0; sb < nslabs; ++sb) {
    const int b = sb & 1;
    if (sb + 1 < nslabs) load(sb + 1);
    u32x4 af[2], bfr[MT];
#pragma unroll
    for (int t = 0; t < 2; ++t) af[t] = *reinterpret_cast<const u32x4*>(&wl[b][slot_of(32 * wave + 16 * t + r, g)]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bfr[mt] = *reinterpret_cast<const u32x4*>(&xl[b][slot_of(16 * mt + r, g)]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const long a8 = (long)(((uint64_t)af[t][2 * j + 1] << 32) | af[t][2 * j]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const long b8 = (long)(((uint64_t)bfr[mt][2 * j + 1] << 32) | bfr[mt][2 * j]);
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, acc[t][mt], 0, 0, 0);
        }
      }
    if (sb + 1 < nslabs) {
      store(b ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = n0 + 32 * wave + 16 * t + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + r;
      if (m >= M || m >= m0 + BM) continue;
      const float sx = xs[m];
      uint16_t* yrow = y + (int64_t)m * N;
      uint32_t o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int nn = min(n + v, N - 1);
        float val = acc[t][mt][v] * sx * ws[nn];
        if (bias != nullptr) val += __uint_as_float((uint32_t)bias[nn] << 16);
        o[v] = f32_to_bf16_rne(val);
      }
      if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<uint2*>(yrow + n) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) yrow[n + v] = (uint16_t)o[v];
      }
    }
  }
}

hipError_t launch_fp8_quant_rows(const void* a, int64_t R, int64_t K, uint8_t* q, float* scales,
                                 hipStream_t stream) {
  const int64_t blocks = std::min<int64_t>((R + 3) / 4, 65536);
  const void* fn = K <= 2048   ? (const void*)fp8_quant_rows_kernel<4>
                   : K <= 4096 ? (const void*)fp8_quant_rows_kernel<8>
                   : K <= 8192 ? (const void*)fp8_quant_rows_kernel<16>
                               : (const void*)fp8_quant_rows_kernel<0>;
  return launch_kernel(fn, dim3((unsigned)blocks), dim3(256), stream, (const uint16_t*)a, R, (int)K, q, scales);
}

template <int MT>
static hipError_t fp8_gemm_launch(const uint8_t* xq, const float* xs, int M, int K, const uint8_t* wq,
                                  const float* ws, int N, const void* bias, void* y, hipStream_t stream) {
  const dim3 grid((N + kFp8Rows - 1) / kFp8Rows, (M + 16 * MT - 1) / (16 * MT));
  return launch_kernel((const void*)fp8_gemm_kernel<MT>, grid, dim3(256), stream, xq, xs, M, K, wq, ws, N,
                       (const uint16_t*)bias, (uint16_t*)y);
}

hipError_t launch_fp8_gemm(const uint8_t* xq, const float* xs, int64_t M, int64_t K, const uint8_t* wq,
                           const float* ws, int64_t N, const void* bias, void* y, hipStream_t stream) {
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (std::min<int64_t>((M + 15) / 16, 8)) {
    case 1: return fp8_gemm_launch<1>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 2: return fp8_gemm_launch<2>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 3: return fp8_gemm_launch<3>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 4: return fp8_gemm_launch<4>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    default: return fp8_gemm_launch<8>(xq, xs, m, k, wq, ws, n, bias, y, stream);
  }
}

}  // namespace nvfp4
