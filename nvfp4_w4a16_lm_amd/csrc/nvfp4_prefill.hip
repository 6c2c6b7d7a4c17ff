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
// gemm_prefill_small_kernel: M > 64 with K % 64 != 0 (ragged K; not a shape
// this path is tuned for).  128 (n) x 128 (m) output tile per 256-thread workgroup,
// 64-k steps.  Each step stages the packed weight tile (4 KiB + scales) and
// the bf16 activation tile in registers, dequantizes the weights to bf16 into
// LDS, and the four wavefronts (2 x 2, 64 x 64 each) run 4 x 4 MFMA tiles.
// VEC: K % 64 == 0 (full k-steps, 16-byte aligned weight rows).
// ---------------------------------------------------------------------------
constexpr int kBN = 128, kBM = 128, kBK = 64, kLdsPitch = kBK + 8;

template <bool VEC>
__global__ __launch_bounds__(256) void gemm_prefill_small_kernel(const uint16_t* __restrict__ x, int M, int K,
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
// gemm_prefill_kernel: M > 64, K % 64 == 0.  256 (n) x 256 (m) output tile
// per 256-thread workgroup, 64-k steps, v_mfma_f32_32x32x16_bf16.
//
// Each wavefront owns a 128 x 128 quarter of the tile: 4 x 4 MFMA tiles of
// 32 x 32, 256 fp32 accumulators per lane.  Per 64-k step the workgroup
// stages the next step's tiles in LDS (double buffered) around this step's
// 64 MFMAs per wavefront: thread t dequantizes weight row n0 + t (64 codes
// -> 64 exact bf16) and copies 8 pieces of the activation tile (each 16 B,
// 8 threads per 128-byte row); the global loads are issued one step ahead.
//
// 32x32x16 operand layout: lane l supplies row/column l % 32 and 8
// consecutive k of k-group l / 32; accumulator v of lane l holds
// D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].  The weight tile is the A
// operand (rows = n), the activation tile the B operand (columns = m).
// The epilogue applies gs and the bias, rounds to bf16, transposes the tile
// through LDS and writes whole 16-byte pieces of y rows.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPT = 256;             // tile rows (n) and columns (m)
constexpr int kPK = 64;              // k per step
constexpr int kPP = kPK + 8;         // bf16 per LDS row of an operand tile
constexpr int kOP = kPT + 8;         // bf16 per LDS row of the output tile

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                              const uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ gs_ptr, int N,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ y, int m_tiles) {
  // [buffer][0 = weight, 1 = activation][row][k]; reused as the output tile at the end
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kPT][kPP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
  const int n0 = nt * kPT, m0 = mt * kPT;
  const int nk = K / kPK;

  // weight loader: thread t -> row n0 + t: 32 packed bytes + 4 scale bytes per step
  const int64_t wrow = min(n0 + tid, N - 1);
  const uint8_t* wp = packed + wrow * (K >> 1);
  const uint8_t* wsp = scales + wrow * (K >> 4);
  // activation loader: thread t -> rows (t >> 3) + 32 i, 16-byte piece t & 7
  const int xc = tid & 7, xr = tid >> 3;

  struct Stage {
    u32x4 w0, w1;
    uint32_t ws;
    u32x4 xv[8];
  };
  auto gload = [&](int kt, Stage& st) __attribute__((always_inline)) {
    const int k0 = kt * kPK;
    st.w0 = load_stream16(wp + k0 / 2);
    st.w1 = load_stream16(wp + k0 / 2 + 16);
    st.ws = *reinterpret_cast<const uint32_t*>(wsp + k0 / 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + xr + 32 * i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(x + (int64_t)min(m, M - 1) * K + k0 + 8 * xc);
      st.xv[i] = m < M ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // dequantize the weight row into 8 pieces of 8 bf16 and store them and the
  // 8 activation pieces into LDS buffer buf
  auto lstore = [&](const Stage& st, int buf) __attribute__((always_inline)) {
    const float sc[4] = {NVFP4_E4M3_TO_F32(st.ws, 0), NVFP4_E4M3_TO_F32(st.ws, 1), NVFP4_E4M3_TO_F32(st.ws, 2),
                         NVFP4_E4M3_TO_F32(st.ws, 3)};
    const uint32_t dw[8] = {st.w0.x, st.w0.y, st.w0.z, st.w0.w, st.w1.x, st.w1.y, st.w1.z, st.w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<bf16x8*>(&lds[buf][0][tid][8 * j]) = dequant8(dw[j], sc[j >> 1]);
      *reinterpret_cast<u32x4*>(&lds[buf][1][xr + 32 * j][8 * xc]) = st.xv[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // The 64 MFMAs of one step, 16 per 16-k sub-step.
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const int row = lane & 31, kg = 8 * (lane >> 5);
#pragma unroll
    for (int k16 = 0; k16 < kPK / 16; ++k16) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][0][128 * wn + 32 * i + row][16 * k16 + kg]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&lds[buf][1][128 * wm + 32 * j + row][16 * k16 + kg]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  // One step ahead: the next step's global loads are issued before this
  // step's MFMAs and land in LDS (the other buffer) after them.
  Stage st;
  gload(0, st);
  lstore(st, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1, st);
    compute(buf);
    if (more) lstore(st, buf ^ 1);
    __syncthreads();
  }

  // epilogue: y[m][n] = bf16(acc * gs + bias[n]) through an LDS tile [m][n]
  const float gs = *gs_ptr;
  uint16_t (*out)[kOP] = reinterpret_cast<uint16_t (*)[kOP]>(&lds[0][0][0][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // accumulators 4q..4q+3 of MFMA row-tile i: 4 consecutive n, shared by the 4 column tiles
      const int nl = 128 * wn + 32 * i + 8 * q + 4 * (lane >> 5);
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias != nullptr) {
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[v] = __uint_as_float((uint32_t)bias[min(n0 + nl + v, N - 1)] << 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = 128 * wm + 32 * j + (lane & 31);
        uint32_t h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = f32_to_bf16_rne(acc[i][j][4 * q + v] * gs + bv[v]);
        *reinterpret_cast<uint2*>(&out[ml][nl]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
  __syncthreads();
#pragma unroll 4
  for (int it = 0; it < kPT * kPT / 8 / 256; ++it) {
    const int lin = it * 256 + tid;
    const int ml = lin >> 5, c = lin & 31;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m >= M || n >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&out[ml][8 * c]);
    uint16_t* dst = y + (int64_t)m * N + n;
    if ((N & 7) == 0 && n + 8 <= N) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&out[ml][8 * c]);
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = hv[e];
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_gemm_prefill(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                               const uint8_t* scales, const float* global_scale, int64_t N,
                               const void* bias, void* y, hipStream_t stream) {
  if (K % kPK != 0) {
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
    return launch_kernel((const void*)gemm_prefill_small_kernel<false>, grid, dim3(256), stream,
                         (const uint16_t*)x, (int)M, (int)K, packed, scales, global_scale, (int)N,
                         (const uint16_t*)bias, (uint16_t*)y);
  }
  const int m_tiles = (int)((M + kPT - 1) / kPT), n_tiles = (int)((N + kPT - 1) / kPT);
  return launch_kernel((const void*)gemm_prefill_kernel, dim3((unsigned)(m_tiles * n_tiles)), dim3(256), stream,
                       (const uint16_t*)x, (int)M, (int)K, packed, scales, global_scale, (int)N,
                       (const uint16_t*)bias, (uint16_t*)y, m_tiles);
}

}  // namespace nvfp4
