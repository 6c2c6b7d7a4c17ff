// Prefill-side W4A16 NVFP4 GEMM for gfx950 (M > 64 activation rows):
// y[M,N] = x[M,K] . dequant(W)^T (+ bias) on bf16 MFMA.
//
// Method: vLLM API docs, quantization.online.lm_head, _LMHeadNvfp4Method.apply
// (weight-only NVFP4 on the platform's W4A16 kernel; activations stay bf16).
// Dequantized weight: E2M1(code) * e4m3(scale) * global_scale.  code * scale
// has at most 6 significant bits, so it is exact in bf16; the kernels feed it
// to bf16 MFMA (fp32 accumulate) and apply the global scale once per output
// in the fp32 epilogue.
//
// MFMA operand roles: the weight tile is the A operand (rows = vocab rows n),
// the activation tile the B operand (columns = rows m of x).  16x16x32
// (small kernel): lane l holds row/column l % 16 and 8 consecutive k of
// k-group l / 16; accumulator v of lane l holds D[4 (l / 16) + v][l % 16].
// 32x32x16 (main kernel): lane l holds row/column l % 32 and 8 k of half
// l / 32; accumulator v holds D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include <type_traits>

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
// gemm_prefill_small_kernel: M > 64 with K % 64 != 0 (K is a multiple of 16;
// not a shape this path is tuned for).  128 (n) x 128 (m) output tile per
// 256-thread workgroup, 64-k steps, the last one partial (16-k blocks past K
// read as zero).  Each step stages the packed weight tile (4 KiB + scales)
// and the bf16 activation tile in registers, dequantizes the weights to bf16
// into LDS, and the four wavefronts (2 x 2, 64 x 64 each) run 4 x 4 MFMA
// tiles.
// ---------------------------------------------------------------------------
constexpr int kBN = 128, kBM = 128, kBK = 64, kLdsPitch = kBK + 8;

__global__ __launch_bounds__(256) void gemm_prefill_small_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                 const uint8_t* __restrict__ packed,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const float* __restrict__ gs_ptr, int N,
                                                                 const uint16_t* __restrict__ bias,
                                                                 uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[kBN * kLdsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kBM * kLdsPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    u32x4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = kw + 8 * j;
      xv[j] = u32x4{0u, 0u, 0u, 0u};
      if (x_ok && kk < K) xv[j] = *reinterpret_cast<const u32x4*>(xrow + kk);
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kPT = 256;             // tile rows (n) and columns (m)
constexpr int kPK = 64;              // k per step
constexpr int kOP = kPT + 8;         // bf16 per LDS row of the output tile
constexpr int kMaxPrefillK = 1 << 21;             // keeps 32-bit buffer offsets in range
constexpr int kWaitVm0 = 0x0F70;                  // s_waitcnt vmcnt(0) alone

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// gemm_prefill_kernel<JT>: M > 64, K % 64 == 0.  256 (n) x 32 JT (m) output
// tile per 256-thread workgroup (one wavefront per SIMD); wavefront w owns
// weight rows 64 w .. 64 w + 63 of the tile and all 32 JT activation rows:
// 2 x JT tiles of v_mfma_f32_32x32x16_bf16, 32 JT fp32 accumulators per lane.
// JT = 8 (256 x 256, every accumulator register) is the main form; the
// narrower forms take the tiles of a last, partial round of workgroups, each
// 256 x 256 tile split over 8 / JT workgroups so that the round fills the GPU.
//
// Nothing passes through registers on its way into LDS: for every 64-k step,
// the bf16 activation tile (32 JT rows x 128 B), the packed weight codes
// (256 rows x 32 B) and the weights' block scales (256 rows x 4 B) are copied
// straight into one buffer of a three-buffer ring (buffer loads with the LDS
// flag for the activations, rows past M reading as zero; global loads with
// the LDS flag for codes and scales, rows past N repeating row N - 1).
// Each wavefront dequantizes the codes of its own 64 rows in registers
// (E2M1 -> fp32 converter, times the E4M3 scale, upper halves packed to
// bf16: exact); every weight is dequantized once per workgroup and never
// stored as bf16.
//
// k order: the dot product does not depend on the order of k, so the 64 k of
// a step are dealt to the MFMAs in the order that makes each lane's weight
// codes contiguous: in sub-step u (0..3), lane half h = l / 32 supplies
// k = 32 h + 8 u .. + 7 for both operands.  A lane's 32 codes of a row are
// then one 16-byte LDS read per step, and its block scales are bytes 2 h and
// 2 h + 1 of the row's four.
//
// Software pipeline, per step s (buffer s % 3; codes of step s in registers):
//   * sub-steps 0..2: 2 JT MFMAs each; between them the activation fragments
//     of the next sub-step are read and its weight fragments dequantized,
//     and the JT + 3 copies of step s + 2 go into buffer (s + 2) % 3, spread
//     over the 6 JT MFMA slots (that buffer was last read by step s - 1,
//     whose reads all finished before step s - 1's barrier);
//   * each wavefront waits for its copies of step s + 1 (those of step s + 2
//     stay in flight), then one barrier: step s + 1 is visible and nobody
//     reads buffer s % 3 any more;
//   * sub-step 3: the codes, scales and first activation fragments of step
//     s + 1 are read and its first weight fragments dequantized.
// Activation rows: unpadded 128 B, 16-byte piece c of row r at slot
// c ^ (r & 7) ^ ((r >> 3) & 1).  Code rows: 32 B, unswizzled (the 8 lanes of
// a read group touch 8 rows 32 B apart: distinct banks).
// ---------------------------------------------------------------------------
constexpr int kDX = 0;                              // buffer layout: activations,
constexpr int kDW = kPT * 128;                      // then codes,
constexpr int kDS = kDW + kPT * 32;                 // then scales
constexpr int kDBuf = kDS + kPT * 4;                // 41 KiB
constexpr int kDRing = 3;
constexpr int kDLds = (kDRing * kDBuf > kPT * kOP * 2) ? kDRing * kDBuf : kPT * kOP * 2;

// s_waitcnt immediate: vmcnt(vm) lgkmcnt(0), expcnt left alone
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | 0x0070; }

// Workgroup barrier that does not drain outstanding copies (__syncthreads
// would also wait for the copies that must stay in flight).  Callers first
// wait for the copies that matter and for their own LDS reads.
__device__ __forceinline__ void dma_ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from buffer `rsrc` at voff + soff into LDS at dst (lane
// l's bytes at dst + 16 l); bytes past the buffer's size read as zero.  (A
// plain function: the builtin inside a kernel template keeps the host pass
// from instantiating the kernel.)
__device__ __forceinline__ void buffer_copy16_lds(__amdgpu_buffer_rsrc_t rsrc, lds_ptr_t dst, uint32_t voff,
                                                  uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
}

struct DCodes {
  u32x4 code[2];     // 32 codes of row tile i (lane half h's 32 k of the step)
  uint32_t sc[2];    // the row's two block scales of that half (bytes 0, 1)
};

// MFMA slot (of the 2 JT per sub-step) after which dequantization pair p
// (0..7; fragment p >> 2, pair p & 3) of the next sub-step is made
template <int JT>
__device__ constexpr int prefill_pair_slot(int p) { return JT == 8 ? 2 * p + 1 : (p * 2 * JT) / 8; }
// slot u * 2 JT + q of sub-steps u = 0..2 after which copy j (of JT + 3) is issued
template <int JT>
__device__ constexpr int prefill_copy_slot(int j) { return (JT == 8 ? 1 : 0) + (j * 6 * JT) / (JT + 3); }

// Tiles are numbered t = nt * m_tiles + mt over 256 x 256 tiles; a launch
// covers tiles t0, t0 + 1, ..., workgroup b taking slice b % (8 / JT) of
// tile t0 + b / (8 / JT).
template <int JT>
__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                  const uint8_t* __restrict__ packed,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ gs_ptr, int N,
                                                                  const uint16_t* __restrict__ bias,
                                                                  uint16_t* __restrict__ y, int m_tiles, int t0) {
  static_assert(JT == 1 || JT == 2 || JT == 4 || JT == 8, "column tiles per workgroup");
  constexpr int kSplit = 8 / JT;
  constexpr int kRows = 32 * JT;                    // activation rows per workgroup
  constexpr int kCopies = JT + 3;                   // copy instructions per wavefront per step
  constexpr int kQ = 2 * JT;                        // MFMAs per sub-step
  constexpr int kWaitCopies = wait_vm_lgkm0(kCopies);   // all but the last step's copies landed
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = t0 + (int)blockIdx.x / kSplit;
  const int mt = t % m_tiles, nt = t / m_tiles;
  const int n0 = nt * kPT, m0 = mt * kPT + ((int)blockIdx.x % kSplit) * kRows;
  if (m0 >= M) return;                              // a slice wholly past M (whole workgroup)
  const int nsteps = K / kPK;
  const int r = lane & 31, h = lane >> 5;

  // activation copies: instruction p of wavefront w fills rows 8 (4 p + w) .. + 7;
  // lane l fills slot l & 7 of row 8 (4 p + w) + (l >> 3), i.e. logical piece
  // (l & 7) ^ (l >> 3) ^ (w & 1)
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)m0 * K), (short)0, min(M - m0, kRows) * K * 2, 0x00020000);
  uint32_t xdv[JT];
#pragma unroll
  for (int p = 0; p < JT; ++p)
    xdv[p] = (uint32_t)((8 * (4 * p + wave) + (lane >> 3)) * K * 2 + 16 * ((lane & 7) ^ (lane >> 3) ^ (wave & 1)));
  // code copies: instruction c of wavefront w fills rows 32 (4 c + w) + (l >> 1), half l & 1
  const uint8_t* csrc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    csrc[c] = packed + (int64_t)min(n0 + 32 * (4 * c + wave) + (lane >> 1), N - 1) * (K >> 1) + 16 * (lane & 1);
  // scale copies: wavefront w fills rows 64 w + l, 4 bytes each
  const uint8_t* ssrc = scales + (int64_t)min(n0 + 64 * wave + lane, N - 1) * (K >> 4);

  // The ring buffer of step st is st % 3; callers pass it as `ph`, a
  // compile-time constant in the unrolled loop below, so that every LDS
  // address is a base plus an immediate offset.
  // copy d (0 .. JT + 2) of step st into ring buffer ph; steps past the last re-read the last
  auto copy_one = [&](int st, int ph, int d) __attribute__((always_inline)) {
    uint8_t* const buf = lds + ph * kDBuf;
    const int sc = min(st, nsteps - 1);
    if (d < JT) {
      buffer_copy16_lds(xres, (lds_ptr_t)(buf + kDX + (4 * d + wave) * 1024), xdv[d], sc * kPK * 2);
    } else if (d < JT + 2) {
      const int c = d - JT;
      __builtin_amdgcn_global_load_lds((const void*)(csrc[c] + 32 * (int64_t)sc),
                                       (lds_ptr_t)(buf + kDW + 1024 * (4 * c + wave)), 16, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds((const void*)(ssrc + 4 * (int64_t)sc), (lds_ptr_t)(buf + kDS + 256 * wave), 4,
                                       0, 0);
    }
  };

  // reads of step st: codes and scales of row tile i (rows 64 w + 32 i + r),
  // activation fragment of column tile j (rows 32 j + r) for sub-step u
  const int wrow = 64 * wave + r;
  const int xt = (r & 7) ^ ((r >> 3) & 1);
  auto read_code = [&](int ph, int i, DCodes& d) __attribute__((always_inline)) {
    const uint8_t* const buf = lds + ph * kDBuf;
    d.code[i] = *reinterpret_cast<const u32x4*>(buf + kDW + (wrow + 32 * i) * 32 + 16 * h);
    d.sc[i] = *reinterpret_cast<const uint16_t*>(buf + kDS + (wrow + 32 * i) * 4 + 2 * h);
  };
  auto read_x = [&](int ph, int j, int u) __attribute__((always_inline)) {
    const uint8_t* const buf = lds + ph * kDBuf;
    return *reinterpret_cast<const bf16x8*>(buf + kDX + (32 * j + r) * 128 + 16 * ((4 * h + u) ^ xt));
  };

  f32x16 acc[2][JT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // operand registers of the current and the next sub-step
  u32x4 wa[2], wb[2];
  bf16x8 xa[JT], xb[JT];
  float wsc[2];
  // pair e of weight fragment i of sub-step u, from codes d, into dst
  auto dequant_pair = [&](const DCodes& d, int i, int u, int e, u32x4& dst) __attribute__((always_inline)) {
    if (e == 0) wsc[i] = (u < 2) ? NVFP4_E4M3_TO_F32(d.sc[i], 0) : NVFP4_E4M3_TO_F32(d.sc[i], 1);
    const uint32_t c = d.code[i][u];
    switch (e) {          // the converter's byte select must be a constant
      case 0: dst[0] = NVFP4_DEQ_PAIR(c, wsc[i], 0); break;
      case 1: dst[1] = NVFP4_DEQ_PAIR(c, wsc[i], 1); break;
      case 2: dst[2] = NVFP4_DEQ_PAIR(c, wsc[i], 2); break;
      default: dst[3] = NVFP4_DEQ_PAIR(c, wsc[i], 3); break;
    }
  };

  // One step st with its codes in cc; fills nc with the codes of step st + 1.
  // MFMA q of a sub-step is tile (i, j) = (q / JT, q % JT).
  auto kstep = [&](int st, auto PH, const DCodes& cc, DCodes& nc) __attribute__((always_inline)) {
    constexpr int ph = decltype(PH)::value;        // ring buffer of step st
    constexpr int ph1 = (ph + 1) % kDRing, ph2 = (ph + 2) % kDRing;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      u32x4(&wcur)[2] = (u & 1) ? wb : wa;
      u32x4(&wnext)[2] = (u & 1) ? wa : wb;
      bf16x8(&xcur)[JT] = (u & 1) ? xb : xa;
      bf16x8(&xnext)[JT] = (u & 1) ? xa : xb;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        acc[q / JT][q % JT] = mfma32x32x16(__builtin_bit_cast(bf16x8, wcur[q / JT]), xcur[q % JT],
                                           acc[q / JT][q % JT]);
        if (q < JT) xnext[q] = read_x(ph, q, u + 1);
#pragma unroll
        for (int p = 0; p < 8; ++p)
          if (prefill_pair_slot<JT>(p) == q) dequant_pair(cc, p >> 2, u + 1, p & 3, wnext[p >> 2]);
#pragma unroll
        for (int j = 0; j < kCopies; ++j)
          if (prefill_copy_slot<JT>(j) == u * kQ + q) copy_one(st + 2, ph2, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitCopies);   // step st + 1 has landed; this wavefront's reads are done
    dma_ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 3 (operands in wb, xb); refill wa, xa with sub-step 0 of step st + 1
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      acc[q / JT][q % JT] = mfma32x32x16(__builtin_bit_cast(bf16x8, wb[q / JT]), xb[q % JT], acc[q / JT][q % JT]);
      if (q == 0) read_code(ph1, 0, nc);
      if (q == (JT == 8 ? 1 : 0)) read_code(ph1, 1, nc);
      if (q < JT) xa[q] = read_x(ph1, q, 0);
      if (JT == 8 && q >= 8) dequant_pair(nc, (q - 8) >> 2, 0, q & 3, wa[(q - 8) >> 2]);
      if (JT < 8 && q == kQ - 1) {
#pragma unroll
        for (int p = 0; p < 8; ++p) dequant_pair(nc, p >> 2, 0, p & 3, wa[p >> 2]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: steps 0 and 1 in flight; step 0 landed; its codes, first
  // activation fragments and first weight fragments in registers
#pragma unroll
  for (int tt = 0; tt < 2 * kCopies; ++tt) copy_one(tt / kCopies, tt / kCopies, tt % kCopies);
  __builtin_amdgcn_s_waitcnt(kWaitCopies);
  dma_ring_barrier();
  DCodes ca, cb;
  read_code(0, 0, ca);
  read_code(0, 1, ca);
#pragma unroll
  for (int j = 0; j < JT; ++j) xa[j] = read_x(0, j, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q) dequant_pair(ca, q >> 2, 0, q & 3, wa[q >> 2]);

  // six steps per iteration: ring buffers 0, 1, 2, 0, 1, 2 and the code
  // registers alternate, all known at compile time; then up to five more
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int st = 0;
  for (; st + 6 <= nsteps; st += 6) {
    kstep(st, I0{}, ca, cb);
    kstep(st + 1, I1{}, cb, ca);
    kstep(st + 2, I2{}, ca, cb);
    kstep(st + 3, I0{}, cb, ca);
    kstep(st + 4, I1{}, ca, cb);
    kstep(st + 5, I2{}, cb, ca);
  }
  if (st < nsteps) kstep(st, I0{}, ca, cb);
  if (st + 1 < nsteps) kstep(st + 1, I1{}, cb, ca);
  if (st + 2 < nsteps) kstep(st + 2, I2{}, ca, cb);
  if (st + 3 < nsteps) kstep(st + 3, I0{}, cb, ca);
  if (st + 4 < nsteps) kstep(st + 4, I1{}, ca, cb);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);            // the last (unused) copies land before LDS is reused
  __syncthreads();

  // epilogue: y[m][n] = bf16(acc * gs + bias[n]) through an LDS tile [m][n]
  const float gs = *gs_ptr;
  uint16_t (*out)[kOP] = reinterpret_cast<uint16_t (*)[kOP]>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // accumulators 4q..4q+3 of MFMA row-tile i: 4 consecutive n, shared by the JT column tiles
      const int nl = 64 * wave + 32 * i + 8 * q + 4 * h;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias != nullptr) {
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[v] = __uint_as_float((uint32_t)bias[min(n0 + nl + v, N - 1)] << 16);
      }
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int ml = 32 * j + r;
        uint32_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[v] = f32_to_bf16_rne(acc[i][j][4 * q + v] * gs + bv[v]);
        *reinterpret_cast<uint2*>(&out[ml][nl]) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    }
  __syncthreads();
#pragma unroll 4
  for (int it = 0; it < kPT * kRows / 8 / 256; ++it) {
    const int lin = it * 256 + tid;
    const int ml = lin >> 5, c = lin & 31;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m >= M || n >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&out[ml][8 * c]);
    uint16_t* dst = y + (int64_t)m * N + n;
    if ((N & 7) == 0 && n + 8 <= N) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));   // logits are not read back here
    } else {
      const uint16_t* hh = reinterpret_cast<const uint16_t*>(&out[ml][8 * c]);
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = hh[e];
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int JT>
static hipError_t launch_prefill_tiles(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                                       const uint8_t* scales, const float* global_scale, int64_t N, const void* bias,
                                       void* y, int m_tiles, int t0, int tiles, hipStream_t stream) {
  return launch_kernel((const void*)gemm_prefill_kernel<JT>, dim3((unsigned)(tiles * (8 / JT))), dim3(256), stream,
                       (const uint16_t*)x, (int)M, (int)K, packed, scales, global_scale, (int)N,
                       (const uint16_t*)bias, (uint16_t*)y, m_tiles, t0);
}

hipError_t launch_gemm_prefill(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                               const uint8_t* scales, const float* global_scale, int64_t N,
                               const void* bias, void* y, hipStream_t stream) {
  if (K % kPK != 0 || K > kMaxPrefillK) {
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
    return launch_kernel((const void*)gemm_prefill_small_kernel, grid, dim3(256), stream,
                         (const uint16_t*)x, (int)M, (int)K, packed, scales, global_scale, (int)N,
                         (const uint16_t*)bias, (uint16_t*)y);
  }
  const int m_tiles = (int)((M + kPT - 1) / kPT), n_tiles = (int)((N + kPT - 1) / kPT);
  const int tiles = m_tiles * n_tiles;
  // One workgroup per compute unit at a time.  Whole rounds of 256 x 256
  // tiles run as they are; the tiles of a last, partial round are split over
  // up to 8 workgroups each so that round keeps every compute unit busy.
  const int cus = device_cus(current_device());
  const int full = tiles / cus * cus;
  const int rest = tiles - full;
  int split = 1;
  while (split < 8 && rest * split * 2 <= cus) split *= 2;
  if (split == 1) {
    return launch_prefill_tiles<8>(x, M, K, packed, scales, global_scale, N, bias, y, m_tiles, 0, tiles, stream);
  }
  if (full > 0) {
    const hipError_t e =
        launch_prefill_tiles<8>(x, M, K, packed, scales, global_scale, N, bias, y, m_tiles, 0, full, stream);
    if (e != hipSuccess) return e;
  }
  switch (split) {
    case 2: return launch_prefill_tiles<4>(x, M, K, packed, scales, global_scale, N, bias, y, m_tiles, full, rest, stream);
    case 4: return launch_prefill_tiles<2>(x, M, K, packed, scales, global_scale, N, bias, y, m_tiles, full, rest, stream);
    default: return launch_prefill_tiles<1>(x, M, K, packed, scales, global_scale, N, bias, y, m_tiles, full, rest, stream);
  }
}

}  // namespace nvfp4
