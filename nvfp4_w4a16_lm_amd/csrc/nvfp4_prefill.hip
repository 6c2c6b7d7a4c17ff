// Prefill-side W4A16 NVFP4 GEMM for gfx950 (M > 64 activation rows):
// y[M,N] = x[M,K] . dequant(W)^T (+ bias) on bf16 MFMA.
//
// Method: vLLM API docs, quantization.online.lm_head, _LMHeadNvfp4Method.apply
// (weight-only NVFP4 on the platform's W4A16 kernel; activations stay bf16).
// Dequantized weight: E2M1(code) * e4m3(scale) * global_scale.  code * scale
// has at most 6 significant bits, so it is exact in bf16; the kernel feeds it
// to bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate) and applies the
// global scale once per output in the fp32 epilogue.
//
// MFMA operand roles: the weight tile is the A operand (16 rows = 16 vocab
// rows n), the activation tile the B operand (16 columns = 16 rows m of x).
// Lane l holds row/column (l % 16) and 8 consecutive k of k-group (l / 16);
// the accumulator lane l holds D[4*(l/16) + v][l % 16], v = 0..3, i.e. four
// consecutive n for one m.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_out(uint16_t* __restrict__ y, const uint16_t* __restrict__ bias,
                                          int64_t m, int64_t n, int64_t N, float acc, float gs) {
  float v = acc * gs;
  if (bias != nullptr) v += __uint_as_float((uint32_t)bias[n] << 16);
  y[m * N + n] = (uint16_t)f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// Prefill: M > 64.  128 (n) x 128 (m) output tile per 256-thread workgroup,
// 64-k steps.  Each step stages the packed weight tile (4 KiB + scales) and
// the bf16 activation tile in registers, dequantizes the weights to bf16 into
// LDS, and the four wavefronts (2 x 2, 64 x 64 each) run 4 x 4 MFMA tiles.
// VEC: K % 64 == 0 (full k-steps, 16-byte aligned weight rows).
// ---------------------------------------------------------------------------
constexpr int kBN = 128, kBM = 128, kBK = 64, kLdsPitch = kBK + 8;

template <bool VEC>
__global__ __launch_bounds__(256) void gemm_prefill_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ gs_ptr, int N,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[kBN * kLdsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kBM * kLdsPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
  const int r = lane & 15, g = lane >> 4;
  const int lrow = tid >> 1, lhalf = tid & 1;   // loader: tile row, 32-k half of the step
  const bool w_ok = n0 + lrow < N, x_ok = m0 + lrow < M;
  const uint8_t* prow = packed + (int64_t)(w_ok ? n0 + lrow : 0) * (K / 2);
  const uint8_t* srow = scales + (int64_t)(w_ok ? n0 + lrow : 0) * (K / 16);
  const uint16_t* xrow = x + (int64_t)(x_ok ? m0 + lrow : 0) * K;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    const int kw = k0 + 32 * lhalf;
    uint32_t pw[4] = {0u, 0u, 0u, 0u};
    uint32_t s01 = 0;
    if (w_ok) {
      if (VEC) {
        const uint4 v = *reinterpret_cast<const uint4*>(prow + kw / 2);
        pw[0] = v.x; pw[1] = v.y; pw[2] = v.z; pw[3] = v.w;
        s01 = (uint32_t)srow[kw / 16] | ((uint32_t)srow[kw / 16 + 1] << 8);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = kw + 16 * j;
          if (kk < K) {
            const uint2 v = *reinterpret_cast<const uint2*>(prow + kk / 2);
            pw[2 * j] = v.x;
            pw[2 * j + 1] = v.y;
            s01 |= (uint32_t)srow[kk / 16] << (8 * j);
          }
        }
      }
    }
    u32x4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = kw + 8 * j;
      xv[j] = u32x4{0u, 0u, 0u, 0u};
      if (x_ok && (VEC || kk < K)) xv[j] = *reinterpret_cast<const u32x4*>(xrow + kk);
    }
    __syncthreads();   // the previous step's fragment reads are done
    const float sv[2] = {NVFP4_E4M3_TO_F32(s01, 0), NVFP4_E4M3_TO_F32(s01, 1)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<bf16x8*>(&Ws[lrow * kLdsPitch + 32 * lhalf + 8 * j]) = dequant8(pw[j], sv[j >> 1]);
      *reinterpret_cast<u32x4*>(&Xs[lrow * kLdsPitch + 32 * lhalf + 8 * j]) = xv[j];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&Ws[(64 * wn + 16 * i + r) * kLdsPitch + kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Xs[(64 * wm + 16 * j + r) * kLdsPitch + kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
  }
  const float gs = *gs_ptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 64 * wm + 16 * j + r;
      if (m >= M) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = n0 + 64 * wn + 16 * i + 4 * g + v;
        if (n < N) store_out(y, bias, m, n, N, acc[i][j][v], gs);
      }
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_gemm_prefill(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                               const uint8_t* scales, const float* global_scale, int64_t N,
                               const void* bias, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  const void* fn = (K % 64 == 0) ? (const void*)gemm_prefill_kernel<true> : (const void*)gemm_prefill_kernel<false>;
  return launch_kernel(fn, grid, dim3(256), stream, (const uint16_t*)x, (int)M, (int)K, packed, scales,
                       global_scale, (int)N, (const uint16_t*)bias, (uint16_t*)y);
}

}  // namespace nvfp4
