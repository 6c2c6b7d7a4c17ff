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
// fp8_prefill_kernel (M > 64, K >= 64, K % 64 == 0): a 256 x 256 output tile per
//   workgroup of 4 wavefronts (2 x 2, 128 x 128 each; 16 MFMAs of
//   v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales per 64-k step,
//   the f8f6f4 form being the one that runs fp8 at the doubled rate; the
//   accumulators of the 4 x 4 tiles in registers).  K is walked in 64-byte
//   steps; both operand tiles (256 rows x 64 bytes each) arrive by
//   direct-to-LDS copies three steps ahead into a ring of four buffers, one
//   copy after every other MFMA of the step before, so each step waits only
//   for its own copies, and one barrier per step both publishes the next
//   tile and frees the buffer the copy after it refills.  Rows are 64 bytes,
//   16-byte piece p of row r at slot p ^ ((r >> 2) & 3).  Lane (r, h) =
//   (l % 32, l / 32) feeds pieces 2 h and 2 h + 1 of its row of each operand
//   (32 k) to each MFMA, the same k order for both operands.  The output
//   tile goes through LDS for row-contiguous 16-byte stores.
#include <algorithm>

#include <type_traits>

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
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

typedef float fp8_f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* fp8_lds_ptr_t;
typedef int fp8_i32x8 __attribute__((ext_vector_type(8)));
constexpr int kFp8UnitScales = 0x7F7F7F7F;           // E8M0 block scales of 1 (2^0) in every byte
constexpr int kFp8WaitVm0 = 0x0F70;                    // s_waitcnt vmcnt(0) alone
constexpr int kFp8PT = 256;                            // prefill tile (rows of each operand)
constexpr int kFp8PStep = kFp8PT * 64;                 // bytes per operand per 64-k step
constexpr int kFp8PBuf = 2 * kFp8PStep;                // one ring buffer: weights, then activations
constexpr int kFp8OP = kFp8PT + 8;                     // bf16 per row of the output staging tile
constexpr int kFp8PRing = 4;                          // ring buffers (copies run 3 steps ahead)
constexpr int kFp8PLds = (kFp8PRing * kFp8PBuf > kFp8PT * kFp8OP * 2) ? kFp8PRing * kFp8PBuf : kFp8PT * kFp8OP * 2;
constexpr int kFp8WaitVm8 = 0x0F78;                    // s_waitcnt vmcnt(8) alone

// Workgroup barrier for the copy ring.  __syncthreads() would also wait for
// every outstanding copy (vmcnt(0)), including the prefetch that must stay in
// flight; here the caller has already waited for the copies that matter, and
// every LDS read before the barrier has been consumed by an MFMA (so its
// lgkmcnt is drained).  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

__global__ __launch_bounds__(256, 1) void fp8_prefill_kernel(const uint8_t* __restrict__ xq,
                                                             const float* __restrict__ xs, int M, int K,
                                                             const uint8_t* __restrict__ wq,
                                                             const float* __restrict__ ws, int N,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ y, int m_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFp8PLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
  const int n0 = nt * kFp8PT, m0 = mt * kFp8PT;
  const int nsteps = K / 64;

  // copies: instruction i of wavefront w fills rows 16 (4 i + w) .. + 15 of an
  // operand tile; lane l fills slot l & 3 of row 16 (4 i + w) + (l >> 2), i.e.
  // piece (l & 3) ^ ((l >> 4) & 3)
  const int cpiece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint8_t* wsrc[4];
  const uint8_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (4 * i + wave) + (lane >> 2);
    wsrc[i] = wq + (int64_t)min(n0 + row, N - 1) * K + 16 * cpiece;
    xsrc[i] = xq + (int64_t)min(m0 + row, M - 1) * K + 16 * cpiece;
  }
  // copy instruction c (0..7) of step st: c < 4 weight rows, c >= 4 activation
  // rows; steps past the last re-read the last step (never used)
  // `ph` is the ring buffer st % 4, a compile-time constant in the unrolled loop
  auto copy_one = [&](int st, int ph, int c) __attribute__((always_inline)) {
    uint8_t* const buf = lds + ph * kFp8PBuf;
    const int64_t off = 64 * (int64_t)min(st, nsteps - 1);
    const int i = c & 3;
    if (c < 4)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + off), (fp8_lds_ptr_t)(buf + 1024 * (4 * i + wave)), 16,
                                       0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(xsrc[i] + off),
                                       (fp8_lds_ptr_t)(buf + kFp8PStep + 1024 * (4 * i + wave)), 16, 0, 0);
  };
  // fragment reads: row 128 wn + 32 i + r of the weight tile, 128 wm + 32 j + r of the activation tile
  const int r = lane & 31, h = lane >> 5;
  auto slot = [&](int row, int p) { return row * 64 + 16 * (p ^ ((row >> 2) & 3)); };
  // the 32 bytes (pieces 2 h, 2 h + 1) of one row that lane half h feeds to a 32x32x64 MFMA
  auto frag32 = [&](const uint8_t* base, int row) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + slot(row, 2 * h));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + slot(row, 2 * h + 1));
    return fp8_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  fp8_f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  typedef fp8_i32x8 Frag[4];
  auto read_frags = [&](int ph, int f, Frag& a, Frag& b) __attribute__((always_inline)) {
    const uint8_t* const wb = lds + ph * kFp8PBuf;
    if (f < 4)
      a[f] = frag32(wb, 128 * wn + 32 * f + r);
    else
      b[f - 4] = frag32(wb + kFp8PStep, 128 * wm + 32 * (f - 4) + r);
  };
  // One k step st (ring buffer PH = st % 4, a compile-time constant): 16
  // MFMAs on the fragments (ca, cb) of step st.  Between them, the fragments
  // of step st + 1 are read into (na, nb) and the copies of step st + 3 are
  // issued, one after every other MFMA, into the buffer step st - 1 used
  // (its fragments were read during step st - 2).  Then the copies of step
  // st + 2 are waited for (the 8 of step st + 3 stay in flight) and the
  // barrier publishes them.
  auto kstep = [&](int st, auto PH, const Frag& ca, const Frag& cb, Frag& na, Frag& nb) __attribute__((always_inline)) {
    constexpr int ph = decltype(PH)::value;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ca[q >> 2], cb[q & 3], acc[q >> 2][q & 3], 0,
                                                                           0, 0, kFp8UnitScales, 0, kFp8UnitScales);
      if (q < 8) read_frags((ph + 1) % kFp8PRing, q, na, nb);
      if (q & 1) copy_one(st + 3, (ph + 3) % kFp8PRing, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kFp8WaitVm8);
    ring_barrier();
  };

  // prologue: steps 0..2 in flight, then steps 0 and 1 landed and step 0's fragments read
#pragma unroll
  for (int c = 0; c < 24; ++c) copy_one(c >> 3, c >> 3, c & 7);
  __builtin_amdgcn_s_waitcnt(kFp8WaitVm8);
  ring_barrier();
  Frag fa, fb, ga, gb;
#pragma unroll
  for (int f = 0; f < 8; ++f) read_frags(0, f, fa, fb);
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  int st = 0;
  for (; st + 4 <= nsteps; st += 4) {
    kstep(st, Q0{}, fa, fb, ga, gb);
    kstep(st + 1, Q1{}, ga, gb, fa, fb);
    kstep(st + 2, Q2{}, fa, fb, ga, gb);
    kstep(st + 3, Q3{}, ga, gb, fa, fb);
  }
  if (st < nsteps) kstep(st, Q0{}, fa, fb, ga, gb);
  if (st + 1 < nsteps) kstep(st + 1, Q1{}, ga, gb, fa, fb);
  if (st + 2 < nsteps) kstep(st + 2, Q2{}, fa, fb, ga, gb);
  __builtin_amdgcn_s_waitcnt(kFp8WaitVm0);           // the last (unused) copies land before LDS is reused
  __syncthreads();                                    // the ring is free for the output tile

  // epilogue: y[m][n] = bf16(acc * s_x[m] * s_w[n] + bias[n]) through an LDS tile [m][n]
  uint16_t (*out)[kFp8OP] = reinterpret_cast<uint16_t (*)[kFp8OP]>(lds);
  float sx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sx[j] = xs[min(m0 + 128 * wm + 32 * j + r, M - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // accumulators 4q..4q+3 of MFMA row-tile i: 4 consecutive n, shared by the 4 column tiles
      const int nl = 128 * wn + 32 * i + 8 * q + 4 * h;
      float sw[4], bv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int nn = min(n0 + nl + v, N - 1);
        sw[v] = ws[nn];
        bv[v] = bias != nullptr ? __uint_as_float((uint32_t)bias[nn] << 16) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = 128 * wm + 32 * j + r;
        uint32_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[v] = f32_to_bf16_rne(acc[i][j][4 * q + v] * sx[j] * sw[v] + bv[v]);
        *reinterpret_cast<uint2*>(&out[ml][nl]) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    }
  __syncthreads();
#pragma unroll 4
  for (int it = 0; it < kFp8PT * kFp8PT / 8 / 256; ++it) {
    const int lin = it * 256 + tid;
    const int ml = lin >> 5, c = lin & 31;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m >= M || n >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&out[ml][8 * c]);
    uint16_t* dst = y + (int64_t)m * N + n;
    if ((N & 7) == 0 && n + 8 <= N) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));   // logits are not read back here
    } else {
      const uint16_t* hvv = reinterpret_cast<const uint16_t*>(&out[ml][8 * c]);
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = hvv[e];
    }
  }
}

// ---------------------------------------------------------------------------
// fp8_ring_kernel<MT, R>: 1 <= M <= 16 MT activation rows (MT = 1, 2, 4),
// K % 512 == 0.  Weights stream through registers, with e4m3 operands and
// nothing to dequantize:
//  * a workgroup of 8 wavefronts owns blocks of 128 R weight rows, R tiles of
//    16 rows per wavefront; a chunk is 128 k (128 bytes of a row); each
//    wavefront keeps two chunks of its tiles in registers in flight, loaded
//    8 lanes per row segment (whole 128-byte lines, nontemporal), and moves
//    each chunk into the operand layout through its own 2 R KiB of LDS
//    (16-byte pieces XOR-swizzled by row, no barrier);
//  * one v_mfma_scale_f32_16x16x128_f8f6f4 per tile, activation tile and
//    chunk (unit block scales; lane (r, g) = (l % 16, l / 16) supplies the
//    32 bytes [32 g, 32 g + 32) of row r of the chunk for both operands);
//  * x is copied into LDS in panels of 32 KiB (pk bytes of 16 MT rows, rows
//    past M repeating row M - 1) by direct-to-LDS loads, double buffered,
//    one workgroup barrier per panel;
//  * loads complete in issue order, so every wait is an exact vmcnt.
// Epilogue: acc * s_x[m] * s_w[n] (+ bias[n]) in float32, one bf16
// rounding.  Rows past N read as zero through the buffer resource and are
// never stored.
// ---------------------------------------------------------------------------
constexpr int kF8RingNW = 8;                           // wavefronts per workgroup (two per SIMD)

template <int MT>
struct F8RingGeom {
  static constexpr int rows = 16 * MT;                          // x rows in a panel
  static constexpr int pk = MT == 1 ? 2048 : MT == 2 ? 1024 : 512;   // panel columns (k = bytes)
  static constexpr int pchunks = pk / 128;                      // chunks per panel: 16, 8, 4
  static constexpr int xbytes = rows * pk;                      // one panel buffer: 32 KiB
  static constexpr int xcopies = xbytes / 1024 / kF8RingNW;     // 1 KiB copies per wavefront per panel
  static_assert(xbytes % (1024 * kF8RingNW) == 0, "panel copies must split evenly over the wavefronts");
  static_assert(pchunks % 4 == 0, "panels start on the unrolled 4-chunk steps");
};

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt bits [3:0] and [15:14])
template <int N>
__device__ __forceinline__ void f8_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

template <int MT, int R, bool kUniform>
__global__ __launch_bounds__(64 * kF8RingNW) void fp8_ring_kernel(const uint8_t* __restrict__ xq,
                                                                const float* __restrict__ xs, int M, int K,
                                                                const uint8_t* __restrict__ wq,
                                                                const float* __restrict__ ws, int N,
                                                                const uint16_t* __restrict__ bias,
                                                                uint16_t* __restrict__ y) {
  using G = F8RingGeom<MT>;
  constexpr int NW = kF8RingNW;
  constexpr int kBatch = 2 * R;                         // loads per chunk
  __shared__ __attribute__((aligned(16))) uint8_t xsl[2][G::xbytes];
  __shared__ __attribute__((aligned(16))) uint8_t wt[NW][R * 2048];
  // the wavefront index is uniform: keeping it in a scalar register keeps the
  // buffer resources below scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = K / 128;
  const int npanels = (K + G::pk - 1) / G::pk;         // the last one partial when K % pk != 0
  // transpose write: load lane l holds row 8 j + l / 8, piece l % 8 (slot piece ^ (row & 7))
  const int wwr = 128 * (lane >> 3) + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
  // operand read: row r, pieces 2 g and 2 g + 1
  const int wrd0 = 128 * r + 16 * ((2 * g) ^ (r & 7)), wrd1 = 128 * r + 16 * ((2 * g + 1) ^ (r & 7));
  uint8_t* const wmine = wt[wave];
  const int wlane = (lane >> 3) * K + 16 * (lane & 7);   // byte offset within this wavefront's rows
  constexpr int kRowsWG = NW * R * 16;
  const int nblocks = (N + kRowsWG - 1) / kRowsWG;

  for (int blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const int n_wave = blk * kRowsWG + wave * (R * 16);
    // rows past N lie outside the resource and read as zero (never stored);
    // every field passes readfirstlane so that the resource stays scalar
    const int rows_in = __builtin_amdgcn_readfirstlane(max(0, min(R * 16, N - n_wave)));
    const int row0 = __builtin_amdgcn_readfirstlane(min(n_wave, N - 1));
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(wq + (int64_t)row0 * K), (short)0, __builtin_amdgcn_readfirstlane(rows_in * K), 0x00020000);

    u32x4 wr[2][R][2];                                  // the ring: chunks c (slot c % 2) and c + 1
    f32x4 acc[R][MT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int c, auto SLOT) {
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wr[decltype(SLOT)::value][t][j] =
              __builtin_amdgcn_raw_buffer_load_b128(wres, wlane + (16 * t + 8 * j) * K, 128 * c, 2 /* nontemporal */);
    };
    // x panel P into buffer b: copy i of this wavefront fills panel bytes [1 KiB (i NW + wave), + 1 KiB);
    // columns past K (a partial last panel) read the row's last 16 (never used)
    auto x_copy = [&](int P, int b) {
      uint8_t* const buf = xsl[b];
#pragma unroll
      for (int i = 0; i < G::xcopies; ++i) {
        const int off = 1024 * (i * NW + wave) + 16 * lane;
        const int m = off / G::pk, slot = (off % G::pk) >> 4;
        const int piece = slot ^ (m & 7);
        const int col = min(P * G::pk + 16 * piece, K - 16);
        __builtin_amdgcn_global_load_lds((const void*)(xq + (int64_t)min(m, M - 1) * K + col),
                                         (fp8_lds_ptr_t)(buf + 1024 * (i * NW + wave)), 16, 0, 0);
      }
    };

    // one chunk; U = c % 4 (the loop below steps c by 4; panels start at U = 0)
    auto step = [&](int c, auto U_) {
      constexpr int u = decltype(U_)::value;
      const int cc = c % G::pchunks;                    // chunk within its panel
      const int P = c / G::pchunks;
      if constexpr (kUniform) {
        // wait for batch(c); batch(c + 1) and, one step after a u = 0 step,
        // the x copies that step issued (after batch(c)) may stay in flight.
        // Every step issues the same loads whatever c is (past the end they
        // repeat the last chunk or panel, never used), so the count of loads
        // issued after each one is fixed, these waits are exact, and the
        // compiler's own waits need not assume the worst.
        if constexpr (u == 1) f8_wait_vmcnt<kBatch + G::xcopies>();
        else f8_wait_vmcnt<kBatch>();
        if constexpr (u == 0) {
          if (cc == 0) asm volatile("s_barrier" ::: "memory");   // panel P is complete; panel P - 1 is no longer read
        }
      } else {
        // wait for batch(c); batch(c + 1) and, after a panel start, the copies
        // of panel P + 1 (issued after batch(c)) may stay in flight
        if (c + 1 < nchunks) {
          if (u == 1 && cc == 1 && P + 1 < npanels) f8_wait_vmcnt<kBatch + G::xcopies>();
          else f8_wait_vmcnt<kBatch>();
        } else {
          f8_wait_vmcnt<0>();
        }
        if constexpr (u == 0) {
          if (cc == 0) {
            asm volatile("s_barrier" ::: "memory");     // panel P is complete; panel P - 1 is no longer read
            if (P + 1 < npanels) x_copy(P + 1, (P + 1) & 1);
          }
        }
      }
      // chunk c: registers -> this wavefront's LDS, then refill the slot with batch(c + 2)
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<u32x4*>(wmine + 2048 * t + 1024 * j + wwr) = wr[u & 1][t][j];
      if constexpr (kUniform) {
        // every u = 0 step copies panel P + 1 into the other buffer (again
        // when not a panel start: the same bytes to the same place; that
        // buffer's panel P - 1 is no longer read after panel P's barrier)
        if constexpr (u == 0) x_copy(min(P + 1, npanels - 1), (P + 1) & 1);
        issue(min(c + 2, nchunks - 1), std::integral_constant<int, u & 1>{});
      } else {
        if (c + 2 < nchunks) issue(c + 2, std::integral_constant<int, u & 1>{});
      }
      fp8_i32x8 bx[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 16 * mt + r;
        const uint8_t* const xr = xsl[P & 1] + row * G::pk;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(xr + 16 * ((8 * cc + 2 * g) ^ (row & 7)));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(xr + 16 * ((8 * cc + 2 * g + 1) ^ (row & 7)));
        bx[mt] = fp8_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(wmine + 2048 * t + wrd0);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(wmine + 2048 * t + wrd1);
        const fp8_i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bx[mt], acc[t][mt], 0, 0, 0, kFp8UnitScales,
                                                                       0, kFp8UnitScales);
        // keep later tiles' operand reads from being hoisted here (register pressure)
        if constexpr (MT >= 2) __builtin_amdgcn_sched_barrier(0);
      }
    };

    x_copy(0, 0);
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});
    for (int c = 0; c < nchunks; c += 4) {
      step(c, std::integral_constant<int, 0>{});
      step(c + 1, std::integral_constant<int, 1>{});
      step(c + 2, std::integral_constant<int, 2>{});
      step(c + 3, std::integral_constant<int, 3>{});
    }

#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int n0 = n_wave + 16 * t + 4 * g;
      float sw[4], bv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int nn = min(n0 + v, N - 1);
        sw[v] = ws[nn];
        bv[v] = bias != nullptr ? __uint_as_float((uint32_t)bias[nn] << 16) : 0.0f;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r;
        if (m >= M) continue;
        const float sx = xs[m];
        uint16_t* yrow = y + (int64_t)m * N;
        uint32_t o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float val = acc[t][mt][v] * sx * sw[v];
          if (bias != nullptr) val += bv[v];
          o[v] = f32_to_bf16_rne(val);
        }
        if ((N & 3) == 0 && n0 + 3 < N) {
          *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n0 + v < N) yrow[n0 + v] = (uint16_t)o[v];
        }
      }
    }
    __syncthreads();                                    // the x buffers are reused by the next block
  }
}

template <int MT, int R, bool kUniform>
static hipError_t fp8_ring_launch(const uint8_t* xq, const float* xs, int M, int K, const uint8_t* wq,
                                  const float* ws, int N, const void* bias, void* y, hipStream_t stream) {
  const void* fn = (const void*)fp8_ring_kernel<MT, R, kUniform>;
  const int nblocks = (N + kF8RingNW * R * 16 - 1) / (kF8RingNW * R * 16);
  const int dev = current_device();
  const dim3 grid(std::min(nblocks, device_cus(dev) * blocks_per_cu(fn, dev, 64 * kF8RingNW, 0)));
  return launch_kernel(fn, grid, dim3(64 * kF8RingNW), stream, xq, xs, M, K, wq, ws, N, (const uint16_t*)bias,
                       (uint16_t*)y);
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

// fp8_dot_kernel<MR, SEG>: M = MR (1 or 2) rows, K % 16 == 0, K <= 1024 SEG.
// VALU dot products: weight rows are dealt in batches of 4 to the wavefronts
// round-robin (wavefront w takes batches w, w + W, ...), two batches in
// flight; lane l covers the 16-byte segments l, l + 64, ... of every row, so
// its slice of the activation rows stays in registers, converted once to
// bf16 pairs.  e4m3 -> bf16 is exact (NVFP4_E4M3X2_TO_BF16), and so is the
// product of two such values in fp32; v_dot2_f32_bf16
// accumulates, a wavefront reduction sums the lanes, and the epilogue is the
// MFMA kernels' (acc * s_x[m] * s_w[n] + bias[n], one bf16 rounding).
// Segments past K hold zero activations, so the clamped weight loads that
// fill them contribute nothing.
template <int MR, int SEG>
__global__ __launch_bounds__(256) void fp8_dot_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      int M, int K, const uint8_t* __restrict__ wq,
                                                      const float* __restrict__ ws, int N,
                                                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                      int nwaves) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r_begin = 4 * wid;
  if (wid >= nwaves || r_begin >= N) return;
  const int rstep = 4 * nwaves;
  const int nseg = K >> 4;

  // this lane's activation slice as bf16 pairs: pair 2 q + h of segment j
  // holds bytes 2 h, 2 h + 1 of word q of the segment's 16 bytes
  bf16x2 xb[MR][SEG][8];
  auto load_batch = [&](int r0, u32x4 (&pk)[4][SEG]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = min(r0 + i, N - 1);       // duplicates are computed, never stored
#pragma unroll
      for (int j = 0; j < SEG; ++j)
        pk[i][j] = load_stream16(wq + row * K + 16 * min(lane + 64 * j, nseg - 1));
    }
  };
  u32x4 pkA[4][SEG], pkB[4][SEG];
  load_batch(r_begin, pkA);                         // the first weights are requested before x
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      const int seg = lane + 64 * j;
      const bool ok = seg < nseg && m < M;
      const u32x4 v = *reinterpret_cast<const u32x4*>(xq + (int64_t)min(m, M - 1) * K + 16 * min(seg, nseg - 1));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wv = ok ? v[q] : 0u;
        xb[m][j][2 * q] = NVFP4_E4M3X2_TO_BF16(wv, false);
        xb[m][j][2 * q + 1] = NVFP4_E4M3X2_TO_BF16(wv, true);
      }
    }
  float sx[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) sx[m] = xs[min(m, M - 1)];

  auto compute_batch = [&](int r0, const u32x4 (&pk)[4][SEG]) {
    float p[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < SEG; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // copy the vector element to a scalar first (see gemv_dot_kernel)
          const uint32_t w = pk[i][j][q];
          const bf16x2 a0 = NVFP4_E4M3X2_TO_BF16(w, false);
          const bf16x2 a1 = NVFP4_E4M3X2_TO_BF16(w, true);
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            p[m][i] = __builtin_amdgcn_fdot2_f32_bf16(a0, xb[m][j][2 * q], p[m][i], false);
            p[m][i] = __builtin_amdgcn_fdot2_f32_bf16(a1, xb[m][j][2 * q + 1], p[m][i], false);
          }
        }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float tot = wave_sum4(p[m], lane);
      const int row = r0 + ((lane >> 5) & 1) * 2 + ((lane >> 4) & 1);
      if ((lane & 15) == 0 && row < N && m < M) {
        float val = tot * sx[m] * ws[row];
        if (bias != nullptr) val += __uint_as_float((uint32_t)bias[row] << 16);
        y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16_rne(val);
      }
    }
  };

  for (int r0 = r_begin; r0 < N; r0 += 2 * rstep) {
    const bool hasB = r0 + rstep < N;
    if (hasB) load_batch(r0 + rstep, pkB);
    compute_batch(r0, pkA);
    if (!hasB) break;
    if (r0 + 2 * rstep < N) load_batch(r0 + 2 * rstep, pkA);
    compute_batch(r0 + rstep, pkB);
  }
}

template <int MR, int SEG>
static hipError_t fp8_dot_launch(const uint8_t* xq, const float* xs, int M, int K, const uint8_t* wq,
                                 const float* ws, int N, const void* bias, void* y, hipStream_t stream) {
  // as many wavefronts as fit at once, trimmed so that each takes the same
  // number of batches (within one)
  const void* fn = (const void*)fp8_dot_kernel<MR, SEG>;
  const int dev = current_device();
  const int resident = 4 * device_cus(dev) * blocks_per_cu(fn, dev, 256, 0);
  const int batches = (N + 3) / 4;
  const int per_wave = (batches + resident - 1) / resident;
  const int waves = (batches + per_wave - 1) / per_wave;
  return launch_kernel(fn, dim3((waves + 3) / 4), dim3(256), stream, xq, xs, M, K, wq, ws, N,
                       (const uint16_t*)bias, (uint16_t*)y, waves);
}

template <int MR>
static hipError_t fp8_dot_dispatch(const uint8_t* xq, const float* xs, int M, int K, const uint8_t* wq,
                                   const float* ws, int N, const void* bias, void* y, hipStream_t stream) {
  switch ((K + 1023) / 1024) {
    case 1: return fp8_dot_launch<MR, 1>(xq, xs, M, K, wq, ws, N, bias, y, stream);
    case 2: return fp8_dot_launch<MR, 2>(xq, xs, M, K, wq, ws, N, bias, y, stream);
    case 3: return fp8_dot_launch<1, 3>(xq, xs, M, K, wq, ws, N, bias, y, stream);   // M = 1 only
    default: return fp8_dot_launch<1, 4>(xq, xs, M, K, wq, ws, N, bias, y, stream);
  }
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
  if (M > 64 && K >= 64 && K % 64 == 0) {
    const int m_tiles = (int)((M + kFp8PT - 1) / kFp8PT), n_tiles = (int)((N + kFp8PT - 1) / kFp8PT);
    return launch_kernel((const void*)fp8_prefill_kernel, dim3((unsigned)(m_tiles * n_tiles)), dim3(256), stream,
                         xq, xs, m, k, wq, ws, n, (const uint16_t*)bias, (uint16_t*)y, m_tiles);
  }
  // one activation row (K <= 4096) or two (K <= 2048: their registers and
  // two batches of weights stay under 256 VGPRs): the VALU dot kernel
  if (K % 16 == 0 && ((M == 1 && K <= 4096) || (M == 2 && K <= 2048))) {
    if (M == 1) return fp8_dot_dispatch<1>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    return fp8_dot_dispatch<2>(xq, xs, m, k, wq, ws, n, bias, y, stream);
  }
  // any other M <= 64 with K % 512 == 0: the register-ring kernel (at one
  // row with K = 8192, 222 against the slab kernel's 241 us; the dot kernel
  // stays ahead where it applies: 95 against 115 us at K = 4096).  The ring
  // kernel's buffer offsets within a wavefront's 64 rows are 32-bit.
  if (K % 512 == 0 && K <= (1 << 24) && M <= 64) {
    // four tiles per wavefront up to 32 rows (two more weight chunks in
    // flight per wavefront); at 64 rows four would spill, so two.  The
    // 17-32-row form issues the same loads every step (120 -> 95 us at the
    // 8B shape, M = 32; it no longer spills); the others measured 2-4 %
    // slower that way and keep their loads conditional.
    if (M <= 16) return fp8_ring_launch<1, 4, false>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    if (M <= 32) return fp8_ring_launch<2, 4, true>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    return fp8_ring_launch<4, 2, false>(xq, xs, m, k, wq, ws, n, bias, y, stream);
  }
  switch (std::min<int64_t>((M + 15) / 16, 8)) {
    case 1: return fp8_gemm_launch<1>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 2: return fp8_gemm_launch<2>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 3: return fp8_gemm_launch<3>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    case 4: return fp8_gemm_launch<4>(xq, xs, m, k, wq, ws, n, bias, y, stream);
    default: return fp8_gemm_launch<8>(xq, xs, m, k, wq, ws, n, bias, y, stream);
  }
}

}  // namespace nvfp4
