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
// gemm_prefill_small_kernel: M > 64 with K % 128 != 0 (not a shape this path
// is tuned for).  128 (n) x 128 (m) output tile per 256-thread workgroup,
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
// gemm_prefill_kernel: M > 64, K % 128 == 0.  256 (n) x 256 (m) output tile
// per 256-thread workgroup (one wavefront per SIMD), 64-k tiles,
// v_mfma_f32_32x32x16_bf16.
//
// Each wavefront owns a 128 x 128 quarter of the tile: 4 x 4 MFMA tiles of
// 32 x 32, 256 fp32 accumulators per lane.  Both operand tiles are staged in
// LDS as bf16, double buffered.
//
// Activation tiles go from global memory straight into LDS (buffer loads with
// the LDS flag; rows past M read as zero): each wavefront instruction fills
// 1 KiB = 8 unpadded 128-byte rows, and the 16-byte pieces of row r are
// stored XOR-swizzled (piece c at slot c ^ (r & 7) ^ ((r >> 3) & 1)) so that
// the fragment reads of 8 (and of 16) consecutive rows hit distinct banks.
//
// Weight tiles are dequantized by the threads: a 64-k tile needs only 32 code
// bytes of each of 256 rows, so rows are read in 128-k superblocks, 4 lanes
// per row (64 contiguous bytes), two superblocks ahead.  Load i of a thread
// covers row n0 + 2 (t >> 2) + (i & 1) + 128 (i >> 1); lane t & 3 takes the
// 16-byte piece (t & 3) ^ 2 (i & 1), so for either 64-k half of a superblock
// every thread holds exactly two pieces (loads {0, 2} or {1, 3}), each 32
// codes of one row and their 2 scale bytes, and writes them to the (padded)
// weight tile.  With this row map the 8 lanes of each LDS store group write 4
// rows with distinct residues mod 4, i.e. distinct banks.
//
// Software pipeline, per 64-k tile kt (LDS buffers b = kt & 1):
//   * 4 sub-steps of 16 k, 16 MFMAs each; the fragments of the next sub-step
//     are read from LDS while the current one's MFMAs run;
//   * between the MFMAs of sub-steps 0..2 the weights of tile kt + 1 are
//     dequantized into weight buffer b ^ 1 (activation tile kt + 1 is already
//     on its way into activation buffer b ^ 1);
//   * one barrier, after sub-step 2's MFMAs (each wavefront first waits for
//     its own activation loads of tile kt + 1): buffer b is no longer read
//     and buffer b ^ 1 is complete, so sub-step 3 runs on registers while the
//     fragments of tile kt + 1 are read and the activation loads of tile
//     kt + 2 into buffer b are issued.
// Loads past the last tile re-read in-bounds data and weight rows past N
// repeat the last row (no branches around loads); those results are never
// stored.
//
// 32x32x16 operand layout: lane l supplies row/column l % 32 and 8
// consecutive k of k-group l / 32; accumulator v of lane l holds
// D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].  The weight tile is the A
// operand (rows = n), the activation tile the B operand (columns = m).
// The epilogue applies gs and the bias, rounds to bf16, transposes the tile
// through LDS and writes whole 16-byte pieces of y rows.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kPT = 256;             // tile rows (n) and columns (m)
constexpr int kPK = 64;              // k per tile
constexpr int kPP = kPK + 8;         // bf16 per LDS row of a weight tile
constexpr int kOP = kPT + 8;         // bf16 per LDS row of the output tile
constexpr int kXBytes = kPT * kPK * 2;            // one activation tile (unpadded)
constexpr int kWBytes = kPT * kPP * 2;            // one weight tile (padded rows)
constexpr int kWBase = 2 * kXBytes;               // LDS: activation buffers 0, 1, then weight buffers 0, 1
constexpr int kLdsBytes = kWBase + 2 * kWBytes;
static_assert(kPT * kOP * 2 <= kLdsBytes, "output tile must fit in the operand buffers");
constexpr int kMaxPrefillK = 1 << 21;             // keeps 32-bit buffer offsets in range
// s_waitcnt immediates (gfx9 encoding): vmcnt(0) / vmcnt(8), other counters not waited for
constexpr int kWaitVm0 = 0x0F70, kWaitVm8 = 0x0F78;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct Frags {
  bf16x8 a[4], b[4];
};

// weight superblock registers of one thread: 4 code pieces and their scale pairs
struct WSuper {
  u32x4 c[4];
  uint32_t s[4];
};

// One tile's 18 weight staging items, in issue order: 0, 1 = select piece 0 / 1;
// 2..17 = half of an 8-weight chunk: id - 2 = 8 piece + 2 chunk + half, where
// half 0 converts code pairs 0, 1 and half 1 pairs 2, 3 and stores the chunk.
__device__ constexpr int kItemOrder[18] = {0, 2, 3, 4, 5, 6, 7, 8, 9, 1, 10, 11, 12, 13, 14, 15, 16, 17};

__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                              const uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ gs_ptr, int N,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ y, int m_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
  const int n0 = nt * kPT, m0 = mt * kPT;
  const int nk = K / kPK;

  // weight loader (see above)
  const int wg = tid >> 2, wj = tid & 3, wa = wj >> 1, wh = wj & 1;
  const uint8_t* wpp[4];
  const uint8_t* wsp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = min(n0 + 2 * wg + (i & 1) + 128 * (i >> 1), N - 1);
    wpp[i] = packed + row * (K >> 1);
    wsp[i] = scales + row * (K >> 4);
  }
  const int kpiece0 = 32 * wj, kpiece1 = 32 * (wj ^ 2);   // k offset in a superblock, loads i even / odd
  auto wsuper_load = [&](int sb, WSuper& w) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ko = min(sb * 2 * kPK + ((i & 1) ? kpiece1 : kpiece0), K - 32);
      w.c[i] = load_stream16(wpp[i] + (ko >> 1));
      w.s[i] = *reinterpret_cast<const uint16_t*>(wsp[i] + (ko >> 4));
    }
  };
  // for half q of a superblock this thread's pieces are loads q ^ wa and (q ^ wa) + 2
  const bool wodd[2] = {wa != 0, wa != 1};

  // activation loader: instruction p of wavefront w fills rows 8 (4 p + w) .. + 7;
  // lane l fills slot l & 7 of row r = 8 (4 p + w) + (l >> 3), i.e. logical
  // piece (l & 7) ^ (r & 7) ^ ((r >> 3) & 1) = (l & 7) ^ (l >> 3) ^ (w & 1)
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)m0 * K), (short)0, min(M - m0, kPT) * K * 2, 0x00020000);
  uint32_t xdv[8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
    xdv[p] = (uint32_t)((8 * (4 * p + wave) + (lane >> 3)) * K * 2 + 16 * ((lane & 7) ^ (lane >> 3) ^ (wave & 1)));
  auto xdma = [&](int kt, int nb, int p) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_ptr_t)(lds + nb * kXBytes + (4 * p + wave) * 1024), 16,
                                             xdv[p], kt * kPK * 2, 0, 0);
  };

  // Per-lane LDS byte offsets.  They pass through an empty asm at the start
  // of every tile so the compiler rebuilds addresses there as base +
  // immediate instead of keeping dozens of loop-invariant addresses live.
  int fw_off = kWBase + ((128 * wn + (lane & 31)) * kPP + 8 * (lane >> 5)) * 2;
  int fx_off[4];
#pragma unroll
  for (int k16 = 0; k16 < 4; ++k16)
    fx_off[k16] = (128 * wm + (lane & 31)) * 128 + 16 * ((2 * k16 + (lane >> 5)) ^ (lane & 7) ^ ((lane >> 3) & 1));
  int ws_off[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
      const int i = (q ^ wa) + 2 * pi;
      ws_off[q][pi] = kWBase + ((2 * wg + (i & 1) + 128 * (i >> 1)) * kPP + 32 * wh) * 2;
    }
  auto launder = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(fw_off), "+v"(fx_off[0]), "+v"(fx_off[1]), "+v"(fx_off[2]), "+v"(fx_off[3]));
    asm volatile("" : "+v"(ws_off[0][0]), "+v"(ws_off[0][1]), "+v"(ws_off[1][0]), "+v"(ws_off[1][1]));
  };
  auto frag_w = [&](int buf, int i, int k16) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(lds + fw_off + buf * kWBytes + i * 32 * kPP * 2 + k16 * 32);
  };
  auto frag_x = [&](int buf, int j, int k16) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(lds + fx_off[k16] + buf * kXBytes + j * 32 * 128);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  WSuper wA, wB;
  u32x4 pc[2];          // selected code pieces
  float psc[2][2];      // their two block scales
  u32x4 dq;             // chunk being converted
  auto stage_item = [&](int id, int q, const WSuper& w, int nb) __attribute__((always_inline)) {
    if (id < 2) {
      const int pi = id;
      const bool o = wodd[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) pc[pi][e] = o ? w.c[2 * pi + 1][e] : w.c[2 * pi][e];
      const uint32_t sp = o ? w.s[2 * pi + 1] : w.s[2 * pi];
      psc[pi][0] = NVFP4_E4M3_TO_F32(sp, 0);
      psc[pi][1] = NVFP4_E4M3_TO_F32(sp, 1);
    } else {
      const int pi = (id - 2) >> 3, c = ((id - 2) >> 1) & 3, half = (id - 2) & 1;
      const uint32_t d = pc[pi][c];
      const float sc = psc[pi][c >> 1];
      if (half == 0) {
        dq[0] = NVFP4_DEQ_PAIR(d, sc, 0);
        dq[1] = NVFP4_DEQ_PAIR(d, sc, 1);
      } else {
        dq[2] = NVFP4_DEQ_PAIR(d, sc, 2);
        dq[3] = NVFP4_DEQ_PAIR(d, sc, 3);
        *reinterpret_cast<u32x4*>(lds + ws_off[q][pi] + nb * kWBytes + 16 * c) = dq;
      }
    }
  };
  // One 16-k sub-step: 16 MFMAs on fc.  After MFMA i: fragment i of the next
  // sub-step (rb, rk16); then weight staging items [it0 + i*n/16,
  // it0 + (i+1)*n/16) of the tile being staged, or (dma) the activation load
  // i - 8 of tile dkt into buffer rb ^ 1.  The compiler may not reorder
  // across the slots.
  auto substep = [&](const Frags& fc, Frags& fn, int rb, int rk16, int it0, int n, int q, const WSuper& w, int nb,
                     bool dma, int dkt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i >> 2][i & 3] = mfma32x32x16(fc.a[i >> 2], fc.b[i & 3], acc[i >> 2][i & 3]);
      if (i < 4)
        fn.a[i] = frag_w(rb, i, rk16);
      else if (i < 8)
        fn.b[i - 4] = frag_x(rb, i - 4, rk16);
      else if (dma)
        xdma(dkt, rb ^ 1, i - 8);
#pragma unroll
      for (int it = it0 + i * n / 16; it < it0 + (i + 1) * n / 16; ++it) stage_item(kItemOrder[it], q, w, nb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  Frags fa, fb;
  // One 64-k tile kt on buffers kt & 1; stages the weights of tile kt + 1
  // (superblock half q of w) and issues the activation loads of tile kt + 2.
  // vm8: 8 weight loads were issued after the activation loads of tile kt + 1
  // (so the wait before the barrier leaves those 8 outstanding)
  auto tile = [&](int kt, int q, const WSuper& w, bool vm8) __attribute__((always_inline)) {
    const int b = kt & 1;
    launder();
    substep(fa, fb, b, 1, 0, 6, q, w, b ^ 1, false, 0);
    substep(fb, fa, b, 2, 6, 6, q, w, b ^ 1, false, 0);
    substep(fa, fb, b, 3, 12, 6, q, w, b ^ 1, false, 0);
    // this wavefront's activation loads of tile kt + 1 have landed; after the
    // barrier every wavefront has read buffer b and filled buffer b ^ 1
    __builtin_amdgcn_sched_barrier(0);
    if (vm8)
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    substep(fb, fa, b ^ 1, 0, 0, 0, q, w, b, true, min(kt + 2, nk - 1));
  };

  // prologue: superblocks 0, 1 and activation tiles 0, 1 in flight; weight tile 0 staged
  wsuper_load(0, wA);
  wsuper_load(1, wB);
#pragma unroll
  for (int p = 0; p < 8; ++p) xdma(0, 0, p);
#pragma unroll
  for (int p = 0; p < 8; ++p) xdma(min(1, nk - 1), 1, p);
#pragma unroll
  for (int it = 0; it < 18; ++it) stage_item(kItemOrder[it], 0, wA, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm8);     // activation tile 0 (tile 1's 8 loads may be pending)
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa.a[i] = frag_w(0, i, 0);
    fa.b[i] = frag_x(0, i, 0);
  }

  // Superblock s lives in wA for even s, wB for odd s: four tiles per pass so
  // that the two register sets never need copying (a copy would wait for
  // loads still in flight).
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    tile(kt, 1, wA, false);           // stages tile kt + 1: superblock kt / 2, second half
    wsuper_load(kt / 2 + 2, wA);
    tile(kt + 1, 0, wB, true);        // tile kt + 2: superblock kt / 2 + 1, first half
    tile(kt + 2, 1, wB, false);       // tile kt + 3: second half
    wsuper_load(kt / 2 + 3, wB);
    tile(kt + 3, 0, wA, true);        // tile kt + 4: superblock kt / 2 + 2, first half
  }
  if (kt < nk) {                      // nk % 4 == 2
    tile(kt, 1, wA, false);
    tile(kt + 1, 0, wB, false);       // stages past the end (never read)
  }
  // the last activation loads (re-reads of the last tile) land before LDS is reused
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // epilogue: y[m][n] = bf16(acc * gs + bias[n]) through an LDS tile [m][n]
  const float gs = *gs_ptr;
  uint16_t (*out)[kOP] = reinterpret_cast<uint16_t (*)[kOP]>(lds);
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
  if (K % (2 * kPK) != 0 || K > kMaxPrefillK) {
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
