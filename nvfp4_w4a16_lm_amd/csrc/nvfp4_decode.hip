// Decode-side W4A16 NVFP4 GEMM for gfx950 (M <= 64 activation rows):
// y[M,N] = x[M,K] . dequant(W)^T (+ bias), streaming the packed weight once.
//
// Method: vLLM API docs, quantization.online.lm_head, _LMHeadNvfp4Method.apply
// (weight-only NVFP4; activations stay bf16).  Dequantized weight:
// E2M1(code) * e4m3(scale) * global_scale; the global scale is applied once
// per output in fp32.
//
// Kernels, all streaming the weights once (0.5625 B per element), chosen by
// launch_gemv from M and K (each is described where it is defined):
//
// gemv_dot_kernel (M <= 2, K % 32 == 0; K <= 8192 at M = 1, 4096 at M = 2): VALU dot
//   products.  One wavefront streams whole rows, each lane a fixed set of
//   16-byte segments (32 k) of every row, so the lane's slice of x stays in
//   registers for the kernel's lifetime.  Per 16-block the E4M3 scale is
//   split into its power of two 2^e and its mantissa mu in [1, 2): the
//   fp4->bf16 converter applies 2^e exactly (it only uses a scale's
//   exponent), v_dot2_f32_bf16 accumulates a block partial, and mu is applied
//   once per block.  About 1.4 VALU ops per weight at M = 1.
// The others run bf16 / f16 MFMA (16x16x32) on weights dequantized in
// registers (code * scale is exact in either type):
// gemv_xres_kernel (3 <= M <= 16 when x fits in LDS): x resident in LDS as
//   f16 rows scaled by a power of two, weights copied straight to LDS.
// gemv_xphase_kernel (3 <= M <= 16 when x does not fit in LDS whole but a
//   range of K / 2, K / 4 or K / 8 columns of it, a multiple of 1024, does):
//   the same with x held one column range at a time and every wavefront's
//   tiles accumulated in registers across the ranges.
// gemv_panel_kernel (other M <= 64, K % 512 == 0): weights copied straight
//   to per-wavefront LDS one chunk ahead, x in LDS panels.
// gemv_mfma_kernel (K % 256 == 0) and gemv_mfma_ragged_kernel (any K % 16
//   == 0): the general forms.
// The x-resident and panel kernels also run the expert layer's grouped GEMM
// on gathered activation rows (kMoe).
#include <type_traits>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {


// s_waitcnt immediates (gfx9 encoding): vmcnt(0) alone / lgkmcnt(0) alone
constexpr int kWaitVm0 = 0x0F70, kWaitLgkm0 = 0xC07F;
constexpr int kCachePolicyNT = 2;   // cache-policy operand of direct-to-LDS loads: nontemporal
constexpr int kScaleGroup = 4;      // chunks of scales per direct-to-LDS scale copy
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t out_bf16(float acc, float gs, const uint16_t* __restrict__ bias, int n) {
  float v = acc * gs;
  if (bias != nullptr) v += __uint_as_float((uint32_t)bias[n] << 16);
  return f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// gemv_dot_kernel<MR, SEG>: M = MR (1 or 2) rows of x; SEG = 16-byte segments
// per lane per row (K <= 2048 * SEG, K % 32 == 0).  The rows are dealt in
// batches of 4: wavefront w of W takes batches w, w + W, w + 2W, ..., so at
// any moment the GPU streams one compact band of rows (measured faster than
// giving each wavefront one contiguous run), with the next batch in flight.
// ---------------------------------------------------------------------------
template <int MR, int SEG>
__global__ __launch_bounds__(256) void gemv_dot_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                       const uint8_t* __restrict__ packed,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gs_ptr, int N,
                                                       const uint16_t* __restrict__ bias,
                                                       uint16_t* __restrict__ y, int nwaves) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r_begin = 4 * wid;
  if (wid >= nwaves || r_begin >= N) return;
  const int r_end = N;
  const int rstep = 4 * nwaves;                     // rows between this wavefront's batches
  const int nseg = K >> 5;
  const int64_t prow = K >> 1, srow = K >> 4;

  // This lane's slice of x: segment j covers k = 32 * (lane + 64 j) .. + 32.
  // Segments past the row end (seg >= nseg) hold zeros, so the duplicate
  // weights the clamped loads below fetch for them contribute nothing.
  // All loads are unconditional (clamped addresses, then a select): a
  // branch around a load makes the compiler wait for it before going on.
  // The first batch of weights is requested before x.
  u32x4 xr[MR][SEG][4];
  auto load_x = [&]() {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int seg = lane + 64 * j;
        const bool ok = (seg < nseg) && (m < M);
        const int64_t base = (int64_t)min(m, M - 1) * K + 32 * min(seg, nseg - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(x + base + 8 * q);
          xr[m][j][q] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
      }
  };
  const float gs = *gs_ptr;

  auto load_batch = [&](int r0, u32x4 (&pk)[4][SEG], uint32_t (&sc)[4][SEG]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = min(r0 + i, r_end - 1);   // duplicates are computed, never stored
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int seg = min(lane + 64 * j, nseg - 1);
        pk[i][j] = load_stream16(packed + row * prow + 16 * seg);
        sc[i][j] = *reinterpret_cast<const uint16_t*>(scales + row * srow + 2 * seg);
      }
    }
  };

  auto compute_batch = [&](int r0, const u32x4 (&pk)[4][SEG], const uint32_t (&sc)[4][SEG]) {
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
        for (int b = 0; b < 2; ++b) {
          const float s = b ? NVFP4_E4M3_TO_F32(sc[i][j], 1) : NVFP4_E4M3_TO_F32(sc[i][j], 0);
          const uint32_t sb = __float_as_uint(s);
          const float e2 = __uint_as_float(sb & 0x7F800000u);                     // 2^e
          const float mu = (s == 0.0f) ? 0.0f : __uint_as_float((sb & 0x807FFFFFu) | 0x3F800000u);
          bf16x2 a[8];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const uint32_t w = pk[i][j][2 * b + d];
            a[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, e2, 0);
            a[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, e2, 1);
            a[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, e2, 2);
            a[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, e2, 3);
          }
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            float blk = 0.0f;
#pragma unroll
            for (int d = 0; d < 2; ++d)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                // copy the vector element to a scalar first: a bit_cast applied
                // directly to an element of an ext_vector lvalue reads element 0
                const uint32_t xe = xr[m][j][2 * b + d][e];
                blk = __builtin_amdgcn_fdot2_f32_bf16(a[4 * d + e], __builtin_bit_cast(bf16x2, xe), blk, false);
              }
            p[m][i] = fmaf(mu, blk, p[m][i]);
          }
        }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float tot = wave_sum4(p[m], lane);
      const int row = r0 + ((lane >> 5) & 1) * 2 + ((lane >> 4) & 1);
      if ((lane & 15) == 0 && row < r_end && m < M)
        y[(int64_t)m * N + row] = (uint16_t)out_bf16(tot, gs, bias, row);
    }
  };

  // Two batches of 4 rows in flight: the next batch loads while this one computes.
  u32x4 pkA[4][SEG], pkB[4][SEG];
  uint32_t scA[4][SEG], scB[4][SEG];
  load_batch(r_begin, pkA, scA);
  load_x();
  for (int r0 = r_begin; r0 < r_end; r0 += 2 * rstep) {
    const bool hasB = r0 + rstep < r_end;
    if (hasB) load_batch(r0 + rstep, pkB, scB);
    compute_batch(r0, pkA, scA);
    if (!hasB) break;
    if (r0 + 2 * rstep < r_end) load_batch(r0 + 2 * rstep, pkA, scA);
    compute_batch(r0 + rstep, pkB, scB);
  }
}

// ---------------------------------------------------------------------------
// gemv_mfma_kernel<MT, R>: MT = ceil(M/16) activation tiles, R weight tiles
// of 16 rows per wavefront, 4 wavefronts per workgroup (64 R rows per block).
//
// HBM streams at full rate only when every load instruction covers whole
// 128-byte lines of a row (measured: ~7.5 TB/s with 8 lanes per row, ~4.5
// TB/s with the 4 lanes per row the MFMA operand layout gives).  So weights
// are loaded 8 lanes per row -- per 256-k chunk, a 16-row tile is two
// instructions of 8 rows x 128 B -- and transposed through a per-wavefront
// LDS region into the operand layout: lane (r, g) = (lane % 16, lane / 16)
// reads row r, bytes [32 g, 32 g + 32) of the chunk, i.e. k = 256 c + 64 g
// + [0, 64); MFMA step s uses k + 8 s .. + 8.  Each lane loads the 4 scale
// bytes of its own k range directly (they are 1/9 of the bytes, and the rest
// of each 128-byte scale line is used by the next 7 chunks).  The chunk of
// x (M rounded up to 16) is staged once per workgroup in double-buffered
// LDS.  Needs K % 256 == 0 (whole lines per row); rows past N are read from
// clamped addresses and their outputs are never stored.
// ---------------------------------------------------------------------------
constexpr int kChunk = 256;
constexpr int kXPitch = kChunk + 8;   // bf16 per LDS row of x (breaks bank alignment)
constexpr int kWPitch = 128 + 16;     // bytes per LDS row of a weight tile

// one wavefront's weights of a 256-k chunk: R tiles x 2 loader pieces, and
// the operand-layout scale word of each tile
template <int R>
struct WChunk {
  u32x4 w[R][2];
  uint32_t s[R];
};

template <int MT, int R>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        const uint8_t* __restrict__ packed,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ gs_ptr, int N,
                                                        const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][16 * MT][kXPitch];
  __shared__ __attribute__((aligned(16))) uint8_t wl[4][R][16][kWPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int lr = lane >> 3, lq = lane & 7;          // loader: row within 8, 16-byte piece of the line
  const int nchunks = (K + kChunk - 1) / kChunk;
  const int64_t prow = K >> 1, srow = K >> 4;
  const int nblocks = (N + 64 * R - 1) / (64 * R);
  const float gs = *gs_ptr;

  for (int rb = blockIdx.x; rb < nblocks; rb += gridDim.x) {
    const int n_base = rb * (64 * R) + wave * (16 * R);
    // loader row pointers: tile t, half j covers rows n_base + 16 t + 8 j + lr
    const uint8_t* lp[R][2];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) lp[t][j] = packed + (int64_t)min(n_base + 16 * t + 8 * j + lr, N - 1) * prow;
    // scale words in operand layout: lane (r, g) of tile t needs the 4 block
    // scales of k = 64 g .. + 64 of row n_base + 16 t + r, i.e. bytes 16 c + 4 g
    const uint8_t* lsc[R];
#pragma unroll
    for (int t = 0; t < R; ++t) lsc[t] = scales + (int64_t)min(n_base + 16 * t + r, N - 1) * srow + 4 * g;
    auto load_w = [&](int c, WChunk<R>& wc) {
      const int64_t off = min((int64_t)128 * c + 16 * lq, prow - 16);
#pragma unroll
      for (int t = 0; t < R; ++t) {
#pragma unroll
        for (int j = 0; j < 2; ++j) wc.w[t][j] = load_stream16(lp[t][j] + off);
        wc.s[t] = *reinterpret_cast<const uint32_t*>(lsc[t] + 16 * min(c, nchunks - 1));
      }
    };
    auto stage = [&](const u32x4 (&v)[R][2], uint8_t (*dst)[16][kWPitch]) {
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&dst[t][8 * j + lr][16 * lq]) = v[t][j];
    };
    // x staging: 16*MT rows x 256 k = 512*MT vectors of 8 bf16, 2*MT per thread.
    auto load_x = [&](int c, u32x4 (&xv)[2 * MT]) {
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        const int v = tid + 256 * i;
        const int m = v >> 5, k = c * kChunk + 8 * (v & 31);
        const u32x4 val = *reinterpret_cast<const u32x4*>(x + (int64_t)min(m, M - 1) * K + min(k, K - 8));
        xv[i] = (m < M && k < K) ? val : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto store_x = [&](int buf, const u32x4 (&xv)[2 * MT]) {
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        const int v = tid + 256 * i;
        *reinterpret_cast<u32x4*>(&xs[buf][v >> 5][8 * (v & 31)]) = xv[i];
      }
    };

    f32x4 acc[R][MT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA step s (k = 64 g + 8 s .. + 8 of the chunk) reads its MT activation
    // fragments once and applies them to all R weight tiles.
    auto compute = [&](const WChunk<R>& wc, int buf) {
      u32x4 wd[R][2];
      float sv[R][4];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        wd[t][0] = *reinterpret_cast<const u32x4*>(&wl[wave][t][r][32 * g]);
        wd[t][1] = *reinterpret_cast<const u32x4*>(&wl[wave][t][r][32 * g + 16]);
        const uint32_t sw = wc.s[t];
        sv[t][0] = NVFP4_E4M3_TO_F32(sw, 0);
        sv[t][1] = NVFP4_E4M3_TO_F32(sw, 1);
        sv[t][2] = NVFP4_E4M3_TO_F32(sw, 2);
        sv[t][3] = NVFP4_E4M3_TO_F32(sw, 3);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 bx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          bx[mt] = *reinterpret_cast<const bf16x8*>(&xs[buf][16 * mt + r][64 * g + 8 * s]);
#pragma unroll
        for (int t = 0; t < R; ++t) {
          const uint32_t w = wd[t][s >> 2][s & 3];
          const bf16x8 a = dequant8(w, sv[t][s >> 1]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(a, bx[mt], acc[t][mt]);
        }
      }
    };

    WChunk<R> wc0, wc1;
    u32x4 xv[2 * MT];
    load_x(0, xv);
    load_w(0, wc0);
    store_x(0, xv);
    __syncthreads();
    // one step: stage chunk c's weights into this wavefront's LDS, compute,
    // stage the prefetched x
    auto step = [&](int c, const WChunk<R>& wcur, WChunk<R>& wnext) {
      const bool has_next = c + 1 < nchunks;
      if (has_next) {
        load_x(c + 1, xv);          // x first: waiting on it must not wait on the weights
        load_w(c + 1, wnext);
      }
      stage(wcur.w, wl[wave]);
      compute(wcur, c & 1);
      if (has_next) store_x((c + 1) & 1, xv);
      __syncthreads();
    };
    for (int c = 0; c < nchunks; c += 2) {
      step(c, wc0, wc1);
      if (c + 1 < nchunks) step(c + 1, wc1, wc0);
    }

#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int n0 = n_base + 16 * t + 4 * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r;
        if (m >= M) continue;
        uint16_t* yrow = y + (int64_t)m * N;
        if ((N & 3) == 0 && n0 + 3 < N) {
          const uint32_t lo = out_bf16(acc[t][mt][0], gs, bias, n0) | (out_bf16(acc[t][mt][1], gs, bias, n0 + 1) << 16);
          const uint32_t hi = out_bf16(acc[t][mt][2], gs, bias, n0 + 2) | (out_bf16(acc[t][mt][3], gs, bias, n0 + 3) << 16);
          *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n0 + v < N) yrow[n0 + v] = (uint16_t)out_bf16(acc[t][mt][v], gs, bias, n0 + v);
        }
      }
    }
  }  // row blocks
}

// ---------------------------------------------------------------------------
// gemv_xres_kernel<NW, kMoe, KS, kDepth>: 2 < M <= 16 with the whole
// activation resident in LDS (M * (2K + 16) bytes; K % 256 == 0).  NW
// wavefronts per workgroup; x is copied into LDS once, then every wavefront
// streams whole 16-row weight tiles over all of K with no further
// synchronisation.  Each 256-k chunk of a tile's weights (and every 4 chunks
// its scales) is copied by direct-to-LDS loads into the wavefront's own
// swizzled regions and read in the 16x16x32 operand layout, as in
// gemv_panel_kernel:
//  * kDepth = 0: one chunk region; the next chunk's copies are issued once
//    the current chunk has been read out of it (across tiles too);
//  * kDepth = D = 2 or 3 (K % 1024 == 0): D chunk regions used in turn;
//    chunk i + D's copies are issued as soon as chunk i has been read,
//    before chunk i is computed, so a wavefront always has the next D chunks
//    in flight (the scale words of a 4-chunk group are read into registers
//    at its first chunk, and the next group's copy goes out D chunks ahead).
// MFMA columns m >= M read row M - 1 of x and are never stored.
//
// The arithmetic is f16 MFMA with fp32 accumulation:
//  * weights: code * s is exact in f16 (at most 6 significant bits, within
//    [2^-10, 2688]).  With s = 2^e * mu (mu in [1, 2), 3 fraction bits),
//    v_cvt_scalef32_pk_f16_fp4 applies 2^e exactly and one packed f16
//    multiply applies mu: 8 VALU ops per 8 weights instead of 20 on the fp32
//    route (exactness checked on the GPU for all code pairs and scales);
//  * activations: row m is stored as x * 2^-p_m in f16, with p_m set from the
//    row's largest |x| so that it lands in [2^14, 2^15).  Every x with
//    |x| >= 2^-28 max|x_m| converts exactly (bf16's 8 significant bits fit);
//    smaller ones become f16 subnormals or zero, an error below
//    2^-38 max|x_m| per element.  The epilogue multiplies by 2^p_m.
// ---------------------------------------------------------------------------
constexpr int kXresLdsMax = 160 * 1024;

// Expert-layer use of gemv_xres_kernel (kMoe): workgroup row blockIdx.y is
// expert e; its activation rows are the expert's pairs order[offsets[e] ..
// offsets[e + 1]) (row p reads x[p / row_div], writes y[p]); experts with
// fewer than mmin (at least 1) or more than mcap pairs are left to the other
// expert kernels.  gemv_panel_kernel takes the same rows.  When zero_group
// is E (the group of pairs whose id lies outside [0, E)), the workgroups of
// row E write zeros to those pairs' rows instead.
struct MoeRows {
  const int32_t* offsets;
  const int32_t* order;
  int row_div;
  int mcap;
  int mmin;
  int zero_group;   // -1: none
};

template <int NW, bool kMoe = false, int KS = 1, int kDepth = 0>
__global__ __launch_bounds__(64 * NW) void gemv_xres_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                          const uint8_t* __restrict__ packed,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ gs_ptr, int N,
                                                          const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ y, MoeRows moe) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int64_t first = 0;
  if constexpr (kMoe) {                               // uniform over the workgroup, before any barrier
    const int e = blockIdx.y;
    first = moe.offsets[e];
    M = moe.offsets[e + 1] - (int)first;
    if (e == moe.zero_group) {                        // pairs with an invalid id: zero rows, this workgroup's tiles
      const int slots = NW / KS, ntiles = (N + 15) / 16;
      for (int t0 = blockIdx.x * slots; t0 < ntiles; t0 += gridDim.x * slots) {
        const int n0 = 16 * t0, cols = min(16 * slots, N - n0);
        for (int i = threadIdx.x; i < M * cols; i += 64 * NW) {
          const int q = i / cols, c = i - q * cols;
          y[(int64_t)moe.order[first + q] * N + n0 + c] = 0;
        }
      }
      return;
    }
    if (M < max(1, moe.mmin) || M > moe.mcap) return;
    packed += (int64_t)e * N * (K >> 1);
    scales += (int64_t)e * N * (K >> 4);
    gs_ptr += e;
  }
  static_assert(kDepth == 0 || (KS == 1 && (kDepth == 2 || kDepth == 3)), "pipeline depth 2 or 3, whole tiles");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xpitch = 2 * K + 16;                    // bytes per x row (the pad spreads rows over banks)
  constexpr int kWBytes = 2048 * (kDepth ? kDepth : 1);   // per wavefront: regions of 16 rows x 128 B of weights
  uint8_t* const xl = lds;
  uint8_t* const wmine = lds + M * xpitch + kWBytes * wave;
  uint8_t* const smine = lds + M * xpitch + kWBytes * NW + 1024 * wave;   // 16 rows x 64 B of scales
  float* const xup = reinterpret_cast<float*>(lds + M * xpitch + (kWBytes + 1024) * NW);   // 2^p_m
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = K / kChunk;
  const int64_t prow = K >> 1, srow = K >> 4;
  // copies: weight piece (lane & 7) ^ (lane >> 3) of row 8 j + (lane >> 3); scale piece
  // (lane & 3) ^ ((lane >> 3) & 3) of row lane >> 2 (the swizzles of gemv_panel_kernel)
  const int wpiece = (lane & 7) ^ (lane >> 3), spiece = (lane & 3) ^ ((lane >> 3) & 3);
  const int wrd0 = r * 128 + 16 * ((2 * g) ^ (r & 7)), wrd1 = r * 128 + 16 * ((2 * g + 1) ^ (r & 7));
  const int srd = r * 64 + 4 * g, skey = (r >> 1) & 3;

  const int ntiles = (N + 15) / 16;
  const int stride = gridDim.x * NW;
  // chunk c of `tile` (rows past N read row N - 1) into weight region `slot`
  auto w_copy = [&](int tile, int c, int slot) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t row = min(16 * tile + 8 * j + (lane >> 3), N - 1);
      __builtin_amdgcn_global_load_lds((const void*)(packed + row * prow + 128 * c + 16 * wpiece),
                                       (lds_ptr_t)(wmine + 2048 * slot + 1024 * j), 16, 0, kCachePolicyNT);
    }
  };
  auto s_copy = [&](int tile, int grp) {
    const int64_t row = min(16 * tile + (lane >> 2), N - 1);
    const int64_t off = min((int64_t)16 * (kScaleGroup * grp + spiece), srow - 16);   // past the row end: unused
    __builtin_amdgcn_global_load_lds((const void*)(scales + row * srow + off), (lds_ptr_t)smine, 16, 0, 0);
  };
  // KS > 1 (expert layer, few tiles): wavefront w works on tile slot w / KS
  // and chunks w % KS, + KS, ... of it; the KS partial tiles are summed
  // through LDS in phase order after each tile round
  const int slots = NW / KS, slot = wave / KS, ph = wave - slot * KS;
  // the first chunk's copies fly while x is converted
  int tile = blockIdx.x * slots + slot;
  if (tile < ntiles && ph < nchunks) {
    if constexpr (kDepth > 0) {                     // scale group 0, chunks 0 .. kDepth - 1
      s_copy(tile, 0);
#pragma unroll
      for (int c = 0; c < kDepth; ++c) w_copy(tile, c, c);
    } else {
      w_copy(tile, ph, 0);
      s_copy(tile, ph / kScaleGroup);
    }
  }

  // x -> f16 rows in LDS: wavefront w handles rows w, w + NW, ...: the row's
  // largest |x| (bf16 magnitudes compare as integers), then x * 2^-p_m.  A
  // row of at most 4096 values is read once, into registers; longer rows
  // are read twice.
  const int xvec = K / 8;                           // 16-byte vectors per x row
  constexpr int kXRegVec = 8;                       // 16-byte vectors per lane held in registers
  for (int m = wave; m < M; m += NW) {
    const uint16_t* xr = x + (kMoe ? (int64_t)(moe.order[first + m] / moe.row_div) : (int64_t)m) * K;
    if (xvec <= 64 * kXRegVec) {
      u32x4 v[kXRegVec];
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < kXRegVec; ++j) {          // clamped, unconditional loads; vectors past the row are zero
        const int kv = lane + 64 * j;
        const u32x4 t = *reinterpret_cast<const u32x4*>(xr + 8 * min(kv, xvec - 1));
        v[j] = kv < xvec ? t : u32x4{0u, 0u, 0u, 0u};
        mx = pk_max_u16(mx, pk_max_u16(pk_max_u16(v[j].x & 0x7FFF7FFFu, v[j].y & 0x7FFF7FFFu),
                                       pk_max_u16(v[j].z & 0x7FFF7FFFu, v[j].w & 0x7FFF7FFFu)));
      }
      mx = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
      const int p = (mx == 0u) ? 0 : max(-126, (int)(mx >> 7) - 141);   // biased exponent - 127 - 14
      const float down = __uint_as_float((uint32_t)(127 - p) << 23);
      if (lane == 0) xup[m] = __uint_as_float((uint32_t)(127 + p) << 23);
#pragma unroll
      for (int j = 0; j < kXRegVec; ++j) {
        const int kv = lane + 64 * j;
        if (kv < xvec) {
          u32x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 pair = {(_Float16)(bf16_lo(v[j][e]) * down), (_Float16)(bf16_hi(v[j][e]) * down)};
            h[e] = __builtin_bit_cast(uint32_t, pair);
          }
          *reinterpret_cast<u32x4*>(xl + m * xpitch + 16 * kv) = h;
        }
      }
      continue;
    }
    uint32_t mx = 0;
    for (int kv = lane; kv < xvec; kv += 64) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * kv);
      mx = pk_max_u16(mx, pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                     pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu)));
    }
    mx = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    const int p = (mx == 0u) ? 0 : max(-126, (int)(mx >> 7) - 141);   // biased exponent - 127 - 14
    const float down = __uint_as_float((uint32_t)(127 - p) << 23);
    if (lane == 0) xup[m] = __uint_as_float((uint32_t)(127 + p) << 23);
    for (int kv = lane; kv < xvec; kv += 64) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * kv);
      u32x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 pair = {(_Float16)(bf16_lo(v[e]) * down), (_Float16)(bf16_hi(v[e]) * down)};
        h[e] = __builtin_bit_cast(uint32_t, pair);
      }
      *reinterpret_cast<u32x4*>(xl + m * xpitch + 16 * kv) = h;
    }
  }
  __syncthreads();
  const float gs = *gs_ptr;
  const float up = xup[min(r, M - 1)];
  const uint8_t* const xrow = xl + min(r, M - 1) * xpitch + 128 * g;   // this lane's k-group, chunk 0

  if constexpr (KS > 1) {
    f32x4* const red = reinterpret_cast<f32x4*>(lds + M * xpitch + (kWBytes + 1024) * NW + 64);   // [NW][64]
    const int kstride = gridDim.x * slots;
    for (int t0 = blockIdx.x * slots; t0 < ntiles; t0 += kstride) {
      tile = t0 + slot;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tile < ntiles) {
        for (int c = ph; c < nchunks; c += KS) {
          __builtin_amdgcn_s_waitcnt(kWaitVm0);      // this chunk's copies have landed
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(wmine + wrd0);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(wmine + wrd1);
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(smine + srd + 16 * ((c % kScaleGroup) ^ skey));
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);    // the regions may now be overwritten
          const int cn = c + KS;
          if (cn < nchunks) {                         // next chunk, or the next tile's first one
            w_copy(tile, cn, 0);
            if (cn / kScaleGroup != c / kScaleGroup) s_copy(tile, cn / kScaleGroup);
          } else if (tile + kstride < ntiles) {
            w_copy(tile + kstride, ph, 0);
            s_copy(tile + kstride, ph / kScaleGroup);
          }
          float e2[4];
          f16x2 mu[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float sb = b == 0 ? NVFP4_E4M3_TO_F32(sw, 0) : b == 1 ? NVFP4_E4M3_TO_F32(sw, 1)
                           : b == 2 ? NVFP4_E4M3_TO_F32(sw, 2) : NVFP4_E4M3_TO_F32(sw, 3);
            split_scale(sb, &e2[b], &mu[b]);
          }
          const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          const uint8_t* const xc = xrow + 2 * kChunk * c;
          f16x8 bx[8];                                // read together: one LDS latency per chunk
#pragma unroll
          for (int s = 0; s < 8; ++s) bx[s] = *reinterpret_cast<const f16x8*>(xc + 16 * s);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc = mfma16x16x32_f16(dequant8_f16(wd[s], e2[s >> 1], mu[s >> 1]), bx[s], acc);
        }
      }
      red[wave * 64 + lane] = acc;
      __syncthreads();                                // every phase of the round is in LDS
      if (ph == 0 && tile < ntiles && r < M) {
        f32x4 tot = red[(slot * KS) * 64 + lane];
#pragma unroll
        for (int q = 1; q < KS; ++q) tot += red[(slot * KS + q) * 64 + lane];
        tot *= up;
        const int n0 = tile * 16 + 4 * g;
        uint16_t* yrow = y + (kMoe ? (int64_t)moe.order[first + r] : (int64_t)r) * N;
        if ((N & 3) == 0 && n0 + 3 < N) {
          const uint32_t lo = out_bf16(tot[0], gs, bias, n0) | (out_bf16(tot[1], gs, bias, n0 + 1) << 16);
          const uint32_t hi = out_bf16(tot[2], gs, bias, n0 + 2) | (out_bf16(tot[3], gs, bias, n0 + 3) << 16);
          *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n0 + v < N) yrow[n0 + v] = (uint16_t)out_bf16(tot[v], gs, bias, n0 + v);
        }
      }
      __syncthreads();                                // the partials are read before the next round
    }
    return;
  }

  // y row block of `tile` from its accumulators (scaled back by 2^p_m)
  auto store_tile = [&](int t, f32x4 acc) __attribute__((always_inline)) {
    if (r < M) {
      acc *= up;
      const int n0 = t * 16 + 4 * g;
      uint16_t* yrow = y + (kMoe ? (int64_t)moe.order[first + r] : (int64_t)r) * N;
      if ((N & 3) == 0 && n0 + 3 < N) {
        const uint32_t lo = out_bf16(acc[0], gs, bias, n0) | (out_bf16(acc[1], gs, bias, n0 + 1) << 16);
        const uint32_t hi = out_bf16(acc[2], gs, bias, n0 + 2) | (out_bf16(acc[3], gs, bias, n0 + 3) << 16);
        *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n0 + v < N) yrow[n0 + v] = (uint16_t)out_bf16(acc[v], gs, bias, n0 + v);
      }
    }
  };
  // 8 MFMAs of one chunk: weight words w0, w1, the chunk's scale word sw, x
  // chunk xc; even and odd MFMAs accumulate into acc[0] and acc[1] (two
  // independent chains).  The fp4 converter takes each block scale itself
  // (it applies the exponent) and one packed multiply the mantissa.
  auto chunk_mfma = [&](const u32x4& w0, const u32x4& w1, uint32_t sw, const uint8_t* xc, f32x4 (&acc)[2])
      __attribute__((always_inline)) {
    float sb[4];
    f16x2 mu[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sb[b] = b == 0 ? NVFP4_E4M3_TO_F32(sw, 0) : b == 1 ? NVFP4_E4M3_TO_F32(sw, 1)
            : b == 2 ? NVFP4_E4M3_TO_F32(sw, 2) : NVFP4_E4M3_TO_F32(sw, 3);
      mu[b] = scale_mantissa_f16(sb[b]);
    }
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    // the chunk's 8 activation fragments are read together, so that one
    // LDS latency is waited for instead of one per MFMA
    f16x8 bx[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) bx[s] = *reinterpret_cast<const f16x8*>(xc + 16 * s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc[s & 1] = mfma16x16x32_f16(dequant8_f16(wd[s], sb[s >> 1], mu[s >> 1]), bx[s], acc[s & 1]);
  };

  if constexpr (kDepth > 0) {
    // Chunk i of this wavefront's sequence (tile, c) lives in region i % D.
    // Its copies were issued D chunks earlier, the scale group of a chunk
    // with c % 4 == 0 with them (at chunk position (4 - D) % 4); the copies
    // issued after them, 2 per chunk plus that scale copy when it falls in
    // between, may stay in flight.
    constexpr int D = kDepth;
    uint32_t swg[4];
    int slot = 0;                                     // i % D
    // this lane's copy sources in the current tile and in the next one
    // (rows clamped to N - 1): per chunk only a constant offset is added
    const uint8_t* wsrc[2][2];
    const uint8_t* ssrc[2];
    auto set_sources = [&](int t, int which) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wsrc[which][j] = packed + (int64_t)min(16 * t + 8 * j + (lane >> 3), N - 1) * prow + 16 * wpiece;
      ssrc[which] = scales + (int64_t)min(16 * t + (lane >> 2), N - 1) * srow;
    };
    auto step = [&](auto P, int t, int c, f32x4 (&acc)[2]) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;          // c % 4
      constexpr int ps = (4 - D) % 4;                // position whose step also copies the next scale group
      constexpr bool s_between = ((p - ps + 4) % 4) >= 1 && ((p - ps + 4) % 4) <= D - 1;
      constexpr int vm = 2 * (D - 1) + (s_between ? 1 : 0);
      __builtin_amdgcn_s_waitcnt((vm & 15) | 0x0F70);
      uint8_t* const wreg = wmine + 2048 * slot;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(wreg + wrd0);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(wreg + wrd1);
      if (p == 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) swg[b] = *reinterpret_cast<const uint32_t*>(smine + srd + 16 * (b ^ skey));
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // the region (and the scales) may now be refilled
      int which = 0, c2 = c + D;                      // chunk i + D (past the last: clamped rows, never read)
      if (c2 >= nchunks) {
        c2 -= nchunks;
        which = 1;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(wsrc[which][j] + 128 * c2),
                                         (lds_ptr_t)(wmine + 2048 * slot + 1024 * j), 16, 0, kCachePolicyNT);
      if (p == ps) {
        const int64_t off = min((int64_t)16 * (kScaleGroup * (c2 / kScaleGroup) + spiece), srow - 16);
        __builtin_amdgcn_global_load_lds((const void*)(ssrc[which] + off), (lds_ptr_t)smine, 16, 0, 0);
      }
      slot = (slot + 1 == D) ? 0 : slot + 1;
      chunk_mfma(w0, w1, swg[p], xrow + 2 * kChunk * c, acc);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    for (; tile < ntiles; tile += stride) {
      set_sources(tile, 0);
      set_sources(tile + stride, 1);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      for (int c = 0; c < nchunks; c += 4) {
        step(P0{}, tile, c, acc);
        step(P1{}, tile, c + 1, acc);
        step(P2{}, tile, c + 2, acc);
        step(P3{}, tile, c + 3, acc);
      }
      store_tile(tile, acc[0] + acc[1]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);            // the trailing copies land before the workgroup ends
    return;
  }

  for (; tile < ntiles; tile += stride) {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int c = 0; c < nchunks; ++c) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);          // this chunk's copies have landed
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(wmine + wrd0);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(wmine + wrd1);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(smine + srd + 16 * ((c % kScaleGroup) ^ skey));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // the regions may now be overwritten
      if (c + 1 < nchunks) {                          // next chunk, or the next tile's first one
        w_copy(tile, c + 1, 0);
        if ((c + 1) % kScaleGroup == 0) s_copy(tile, (c + 1) / kScaleGroup);
      } else if (tile + stride < ntiles) {
        w_copy(tile + stride, 0, 0);
        s_copy(tile + stride, 0);
      }
      chunk_mfma(w0, w1, sw, xrow + 2 * kChunk * c, acc);
    }
    store_tile(tile, acc[0] + acc[1]);
  }
}

// ---------------------------------------------------------------------------
// gemv_xphase_kernel<NW, TW>: 2 < M <= 16 when the activation does not fit in
// LDS whole but one of its column ranges of kp columns (a phase) does;
// K % kp == 0, kp % 1024 == 0.  The arithmetic, LDS layouts and two-region
// copy pipeline of gemv_xres_kernel, with K walked phase by phase:
//  * wavefront w of workgroup b owns tiles b NW + w + i NW gridDim (i < TW)
//    and keeps the accumulators of all of them in registers;
//  * in phase q it streams chunks q cpp .. q cpp + cpp - 1 (cpp = kp / 256)
//    of each of its tiles in turn; chunk copies run two chunks ahead of its
//    sequence across tile and phase boundaries;
//  * before each phase the workgroup converts that phase's columns of x into
//    LDS (f16, scaled by the 2^-p_m taken from the whole row), between two
//    barriers.
// ---------------------------------------------------------------------------
template <int NW, int TW, int D>
__global__ __launch_bounds__(64 * NW) void gemv_xphase_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                            const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ gs_ptr, int N,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int kp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  static_assert(D == 2 || D == 3, "two or three chunk regions per wavefront");
  constexpr int kRowsPerWave = (16 + NW - 1) / NW;  // x rows each wavefront converts
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xpitch = 2 * kp + 16;                   // bytes per x row of a phase
  uint8_t* const xl = lds;
  uint8_t* const wmine = lds + M * xpitch + 2048 * D * wave;
  uint8_t* const smine = lds + M * xpitch + 2048 * D * NW + 1024 * wave;   // 16 rows x 64 B of scales
  float* const xup = reinterpret_cast<float*>(lds + M * xpitch + (2048 * D + 1024) * NW);   // 2^p_m
  const int r = lane & 15, g = lane >> 4;
  const int cpp = kp / kChunk;                      // chunks per phase, a multiple of 4
  const int nphases = K / kp;
  const int64_t prow = K >> 1, srow = K >> 4;
  const int wpiece = (lane & 7) ^ (lane >> 3), spiece = (lane & 3) ^ ((lane >> 3) & 3);
  const int wrd0 = r * 128 + 16 * ((2 * g) ^ (r & 7)), wrd1 = r * 128 + 16 * ((2 * g + 1) ^ (r & 7));
  const int srd = r * 64 + 4 * g, skey = (r >> 1) & 3;
  const int ntiles = (N + 15) / 16;
  const int stride = gridDim.x * NW;
  const int tile0 = blockIdx.x * NW + wave;
  const int nt = tile0 < ntiles ? min(TW, (ntiles - 1 - tile0) / stride + 1) : 0;   // this wavefront's tiles

  // copies of the chunk at sequence position (phase q, tile i, chunk cc of
  // the phase) into region `slot`, with its scale group when `with_scales`;
  // positions past the end copy the last chunk again (never read)
  auto copy_pos = [&](int q, int i, int cc, int slot, bool with_scales) __attribute__((always_inline)) {
    if (q >= nphases) {
      q = nphases - 1;
      i = nt - 1;
      cc = cpp - 1;
    }
    const int t = tile0 + i * stride;
    const int c = q * cpp + cc;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t row = min(16 * t + 8 * j + (lane >> 3), N - 1);
      __builtin_amdgcn_global_load_lds((const void*)(packed + row * prow + 128 * c + 16 * wpiece),
                                       (lds_ptr_t)(wmine + 2048 * slot + 1024 * j), 16, 0, kCachePolicyNT);
    }
    if (with_scales) {
      const int64_t row = min(16 * t + (lane >> 2), N - 1);
      const int64_t off = min((int64_t)16 * (kScaleGroup * (c / kScaleGroup) + spiece), srow - 16);
      __builtin_amdgcn_global_load_lds((const void*)(scales + row * srow + off), (lds_ptr_t)smine, 16, 0, 0);
    }
  };
  // the position D chunks ahead of the current one, advanced once per chunk
  int qa = 0, ia = 0, ca = 0;
  auto advance = [&]() __attribute__((always_inline)) {
    if (++ca == cpp) {
      ca = 0;
      if (++ia == nt) {
        ia = 0;
        ++qa;
      }
    }
  };
  if (nt > 0) {                                     // the first D chunks fly while x is read
#pragma unroll
    for (int c = 0; c < D; ++c) copy_pos(0, 0, c, c, c == 0);
    ca = D;
  }

  // row scales from the whole row (bf16 magnitudes compare as integers):
  // wavefront w takes rows w, w + NW, ...
  float down[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int m = wave + NW * j;
    down[j] = 1.0f;
    if (m < M) {
      const uint16_t* xr = x + (int64_t)m * K;
      uint32_t mx = 0;
      for (int kv = lane; kv < K / 8; kv += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * kv);
        mx = pk_max_u16(mx, pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                       pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu)));
      }
      mx = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
      const int p = (mx == 0u) ? 0 : max(-126, (int)(mx >> 7) - 141);   // biased exponent - 127 - 14
      down[j] = __uint_as_float((uint32_t)(127 - p) << 23);
      if (lane == 0) xup[m] = __uint_as_float((uint32_t)(127 + p) << 23);
    }
  }

  const uint8_t* const xrow = xl + min(r, M - 1) * xpitch + 128 * g;   // this lane's k-group, chunk 0 of a phase
  f32x4 acc[TW][2];
#pragma unroll
  for (int i = 0; i < TW; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t swg[4];
  int slot = 0;
  // one chunk (cc % 4 == P) of the current tile: wait for its copies (those
  // of the next D - 1 chunks, and the next scale group when its copy went out
  // after them, may stay in flight), read it, refill the region with the
  // chunk D ahead (with its scale group when that chunk starts one, i.e. at
  // P == ps), then 8 MFMAs
  auto step = [&](auto P, int cc, f32x4 (&a)[2]) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    constexpr int ps = (4 - D) % 4;
    constexpr bool s_between = ((p - ps + 4) % 4) >= 1 && ((p - ps + 4) % 4) <= D - 1;
    constexpr int vm = 2 * (D - 1) + (s_between ? 1 : 0);
    __builtin_amdgcn_s_waitcnt((vm & 15) | 0x0F70);
    uint8_t* const wreg = wmine + 2048 * slot;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(wreg + wrd0);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(wreg + wrd1);
    if (p == 0) {
#pragma unroll
      for (int b = 0; b < 4; ++b) swg[b] = *reinterpret_cast<const uint32_t*>(smine + srd + 16 * (b ^ skey));
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);        // the region (and the scales) may now be refilled
    copy_pos(qa, ia, ca, slot, p == ps);
    advance();
    slot = (slot + 1 == D) ? 0 : slot + 1;
    const uint32_t sw = swg[p];
    float sb[4];
    f16x2 mu[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sb[b] = b == 0 ? NVFP4_E4M3_TO_F32(sw, 0) : b == 1 ? NVFP4_E4M3_TO_F32(sw, 1)
            : b == 2 ? NVFP4_E4M3_TO_F32(sw, 2) : NVFP4_E4M3_TO_F32(sw, 3);
      mu[b] = scale_mantissa_f16(sb[b]);
    }
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint8_t* const xc = xrow + 2 * kChunk * cc;
    f16x8 bx[8];                                    // read together: one LDS latency per chunk
#pragma unroll
    for (int s = 0; s < 8; ++s) bx[s] = *reinterpret_cast<const f16x8*>(xc + 16 * s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s & 1] = mfma16x16x32_f16(dequant8_f16(wd[s], sb[s >> 1], mu[s >> 1]), bx[s], a[s & 1]);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;

  for (int q = 0; q < nphases; ++q) {
    __syncthreads();                                // phase q - 1's x is no longer read
    // phase q's columns of x -> f16 rows x * 2^-p_m
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int m = wave + NW * j;
      if (m < M) {
        const uint16_t* xr = x + (int64_t)m * K + (int64_t)q * kp;
        for (int kv = lane; kv < kp / 8; kv += 64) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * kv);
          u32x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 pair = {(_Float16)(bf16_lo(v[e]) * down[j]), (_Float16)(bf16_hi(v[e]) * down[j])};
            h[e] = __builtin_bit_cast(uint32_t, pair);
          }
          *reinterpret_cast<u32x4*>(xl + m * xpitch + 16 * kv) = h;
        }
      }
    }
    __syncthreads();                                // phase q's x is in LDS
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      if (i < nt) {
        for (int cc = 0; cc < cpp; cc += 4) {
          step(P0{}, cc, acc[i]);
          step(P1{}, cc + 1, acc[i]);
          step(P2{}, cc + 2, acc[i]);
          step(P3{}, cc + 3, acc[i]);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);            // the trailing copies land before the workgroup ends

  const float gs = *gs_ptr;
  const float up = xup[min(r, M - 1)];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (i < nt && r < M) {
      const f32x4 tot = (acc[i][0] + acc[i][1]) * up;
      const int n0 = (tile0 + i * stride) * 16 + 4 * g;
      uint16_t* yrow = y + (int64_t)r * N;
      if ((N & 3) == 0 && n0 + 3 < N) {
        const uint32_t lo = out_bf16(tot[0], gs, bias, n0) | (out_bf16(tot[1], gs, bias, n0 + 1) << 16);
        const uint32_t hi = out_bf16(tot[2], gs, bias, n0 + 2) | (out_bf16(tot[3], gs, bias, n0 + 3) << 16);
        *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n0 + v < N) yrow[n0 + v] = (uint16_t)out_bf16(tot[v], gs, bias, n0 + v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemv_panel_kernel<MT, NW, R>: 2 < M <= 64 when the activation does not fit
// in LDS whole; K % 512 == 0.  A workgroup of NW wavefronts owns blocks of
// 16 NW R weight rows (R tiles of 16 rows per wavefront; 8 x 4 is used: two
// wavefronts per SIMD) with the accumulators of the whole block in registers,
// and walks K in panels of `pk` columns:
//  * each panel of x (M rows x pk bf16, at most 64 KiB) is copied into LDS
//    once per workgroup by direct-to-LDS loads, between two barriers;
//  * each 256-k chunk of a wavefront's 16 R weight rows is copied by
//    direct-to-LDS loads (nontemporal) into the wavefront's own 2 R KiB
//    region, 8 rows x 128 B per instruction, one chunk ahead;
//  * every 4 chunks, the 64 scale bytes of each of those rows are copied the
//    same way into a 64 R-byte-per-row region (the scale lines would otherwise
//    be fetched 16 bytes at a time and evicted by the weight stream between
//    uses);
//  * the activation fragments of each MFMA step serve all R tiles.
// LDS rows are unpadded; 16-byte pieces are XOR-swizzled by row so that the
// operand-layout reads hit distinct banks: weight piece q of row j at slot
// q ^ (j & 7), x piece q of row m at q ^ (m & 7), scale piece q of row j at
// q ^ ((j >> 1) & 3).  Rows past N are copied from row N - 1 and never
// stored; MFMA columns past M read row M - 1 of x and are never stored.
// ---------------------------------------------------------------------------
constexpr int kPanelXBytes = 64 * 1024;                 // x panel: M * 2 pk bytes at most

template <int MT, int NW, int kPanelR, bool kMoe = false>
__global__ __launch_bounds__(64 * NW) void gemv_panel_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                         const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ gs_ptr, int N,
                                                         const uint16_t* __restrict__ bias,
                                                         uint16_t* __restrict__ y, int pk, MoeRows moe) {
  int64_t first = 0;
  if constexpr (kMoe) {                               // uniform over the workgroup, before any barrier
    const int e = blockIdx.y;
    first = moe.offsets[e];
    M = moe.offsets[e + 1] - (int)first;
    if (e == moe.zero_group) {                        // pairs with an invalid id: zero rows, this workgroup's blocks
      constexpr int kBlockRows = NW * 16 * kPanelR;
      for (int n0 = blockIdx.x * kBlockRows; n0 < N; n0 += gridDim.x * kBlockRows) {
        const int cols = min(kBlockRows, N - n0);
        for (int i = threadIdx.x; i < M * cols; i += 64 * NW) {
          const int q = i / cols, c = i - q * cols;
          y[(int64_t)moe.order[first + q] * N + n0 + c] = 0;
        }
      }
      return;
    }
    if (M < max(1, moe.mmin) || M > moe.mcap) return;
    packed += (int64_t)e * N * (K >> 1);
    scales += (int64_t)e * N * (K >> 4);
    gs_ptr += e;
    // the widest panel that a pass over the expert's rows (at most 16 MT) fits
    pk = min(K, (kPanelXBytes / min(M, 16 * MT) / 2) / 512 * 512);
  }
  // expert layer (MT <= 2): more than 16 MT pairs are taken in passes of 16 MT rows over each weight block
  const int m_all = M;
  const int64_t first_all = first;
  static_assert(kPanelXBytes >= 16 * MT * 512 * 2, "a panel must hold 512 columns of 16 MT rows");
  constexpr int kRows = 16 * kPanelR;                   // weight rows per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t xp[kPanelXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wl[NW][kRows * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sl[NW][kRows * 16 * kScaleGroup];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = K / kChunk, pchunks = pk / kChunk;
  const int npanels = (nchunks + pchunks - 1) / pchunks;
  const int xpitch = 2 * pk;
  const int64_t prow = K >> 1, srow = K >> 4;
  const float gs = *gs_ptr;
  const int nblocks = (N + NW * kRows - 1) / (NW * kRows);
  // weight copy: lane fills slot lane & 7 of row 8 j + (lane >> 3), i.e. piece (lane & 7) ^ (lane >> 3)
  const int wpiece = (lane & 7) ^ (lane >> 3);
  // operand reads: row 16 t + r, pieces 2 g and 2 g + 1
  const int wrd0 = r * 128 + 16 * ((2 * g) ^ (r & 7)), wrd1 = r * 128 + 16 * ((2 * g + 1) ^ (r & 7));
  // scale copy: lane fills slot lane & 3 of row 16 i + (lane >> 2), i.e. piece (lane & 3) ^ ((lane >> 3) & 3)
  const int spiece = (lane & 3) ^ ((lane >> 3) & 3);
  const int skey = (r >> 1) & 3;                        // scale swizzle of rows 16 t + r
  uint8_t* const wmine = wl[wave];
  uint8_t* const smine = sl[wave];

  constexpr bool kPasses = kMoe && MT <= 2;             // the 64-row form takes at most 64 pairs (one pass)
  for (int blk = blockIdx.x; blk < nblocks; blk += gridDim.x)
  for (int m_pass = 0; m_pass < (kPasses ? m_all : 1); m_pass += 16 * MT) {
    if constexpr (kPasses) {
      M = min(16 * MT, m_all - m_pass);
      first = first_all + m_pass;
    }
    const int n_wave = blk * (NW * kRows) + wave * kRows;
    auto w_copy = [&](int c) {
#pragma unroll
      for (int j = 0; j < kRows / 8; ++j) {
        const int64_t row = min(n_wave + 8 * j + (lane >> 3), N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(packed + row * prow + 128 * c + 16 * wpiece),
                                         (lds_ptr_t)(wmine + 1024 * j), 16, 0, kCachePolicyNT);
      }
    };
    auto s_copy = [&](int grp) {                        // scales of chunks 4 grp .. 4 grp + 3
      const int64_t off = min((int64_t)16 * (kScaleGroup * grp + spiece), srow - 16);   // past the row end: unused
#pragma unroll
      for (int i = 0; i < kRows / 16; ++i) {
        const int64_t row = min(n_wave + 16 * i + (lane >> 2), N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(scales + row * srow + off),
                                         (lds_ptr_t)(smine + 1024 * i), 16, 0, 0);
      }
    };
    auto x_copy = [&](int p) {
      const int per_row = min(pk, K - p * pk) / 512;   // 1 KiB copies per row of this panel
      for (int i = wave; i < M * per_row; i += NW) {
        const int m = i / per_row, h = i - m * per_row;
        const int piece = 64 * h + (lane ^ (m & 7));
        const int64_t xm = kMoe ? (int64_t)(moe.order[first + m] / moe.row_div) : (int64_t)m;
        __builtin_amdgcn_global_load_lds((const void*)(x + xm * K + p * pk + 8 * piece),
                                         (lds_ptr_t)(xp + m * xpitch + 1024 * h), 16, 0, 0);
      }
    };

    f32x4 acc[kPanelR][MT];
#pragma unroll
    for (int t = 0; t < kPanelR; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int xrow[MT], xkey[MT];                             // LDS row offsets and swizzle keys of this lane's x rows

    // chunk c (local chunk cc of the panel); its weights are in wmine and its
    // scales in smine, both copied while the previous chunk computed
    auto chunk = [&](int c, int cc) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);            // this chunk's copies have landed
      u32x4 wd[kPanelR][2];
      uint32_t sw[kPanelR];
      const int c4 = c % kScaleGroup;
#pragma unroll
      for (int t = 0; t < kPanelR; ++t) {
        wd[t][0] = *reinterpret_cast<const u32x4*>(wmine + 2048 * t + wrd0);
        wd[t][1] = *reinterpret_cast<const u32x4*>(wmine + 2048 * t + wrd1);
        sw[t] = *reinterpret_cast<const uint32_t*>(smine + 64 * (16 * t + r) + 16 * (c4 ^ skey) + 4 * g);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);          // the regions may now be overwritten
      if (c + 1 < nchunks) {
        w_copy(c + 1);
        if (c4 == kScaleGroup - 1) s_copy((c + 1) / kScaleGroup);
      }
      // activation fragments one step ahead: step s + 1's LDS reads are in
      // flight while step s's MFMAs issue
      bf16x8 bx[2][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        bx[0][mt] = *reinterpret_cast<const bf16x8*>(xp + xrow[mt] + 512 * cc + 16 * (0 ^ xkey[mt]));
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s + 1 < 8) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            bx[(s + 1) & 1][mt] =
                *reinterpret_cast<const bf16x8*>(xp + xrow[mt] + 512 * cc + 16 * ((s + 1) ^ xkey[mt]));
          __builtin_amdgcn_sched_barrier(0);           // keep them ahead of this step's MFMAs
        }
#pragma unroll
        for (int t = 0; t < kPanelR; ++t) {
          const float sv = (s >> 1) == 0 ? NVFP4_E4M3_TO_F32(sw[t], 0) : (s >> 1) == 1 ? NVFP4_E4M3_TO_F32(sw[t], 1)
                         : (s >> 1) == 2 ? NVFP4_E4M3_TO_F32(sw[t], 2) : NVFP4_E4M3_TO_F32(sw[t], 3);
          const bf16x8 a = dequant8(wd[t][s >> 2][s & 3], sv);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(a, bx[s & 1][mt], acc[t][mt]);
        }
      }
    };

    w_copy(0);
    s_copy(0);
    int c = 0;
    for (int p = 0; p < npanels; ++p) {
      __syncthreads();                                  // the previous panel's reads are done
      x_copy(p);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();                                  // the panel is in LDS
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = min(16 * mt + r, M - 1);
        xrow[mt] = m * xpitch + 128 * g;
        xkey[mt] = m & 7;
      }
      const int c0 = c, c1 = min(nchunks, c + pchunks);
      for (; c < c1; ++c) chunk(c, c - c0);
    }

#pragma unroll
    for (int t = 0; t < kPanelR; ++t) {
      const int n0 = n_wave + 16 * t + 4 * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r;
        if (m >= M) continue;
        uint16_t* yrow = y + (kMoe ? (int64_t)moe.order[first + m] : (int64_t)m) * N;
        if ((N & 3) == 0 && n0 + 3 < N) {
          const uint32_t lo = out_bf16(acc[t][mt][0], gs, bias, n0) | (out_bf16(acc[t][mt][1], gs, bias, n0 + 1) << 16);
          const uint32_t hi = out_bf16(acc[t][mt][2], gs, bias, n0 + 2) | (out_bf16(acc[t][mt][3], gs, bias, n0 + 3) << 16);
          *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n0 + v < N) yrow[n0 + v] = (uint16_t)out_bf16(acc[t][mt][v], gs, bias, n0 + v);
        }
      }
    }
    __syncthreads();                                    // the x region is reused by the next pass or block
  }
}

// ---------------------------------------------------------------------------
// gemv_mfma_ragged_kernel<MT>: the same MFMA arithmetic for K % 256 != 0,
// where rows are not whole 128-byte lines.  One wavefront per 16 rows, the x
// chunk staged in LDS per workgroup, and per-block 8-byte weight loads from
// clamped addresses; blocks past the row end get scale 0.  Kept simple: ragged
// K does not occur in the lm_head shapes this path is tuned for.
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(256) void gemv_mfma_ragged_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                               const uint8_t* __restrict__ packed,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ gs_ptr, int N,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * MT][kXPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int n_base = blockIdx.x * 64 + wave * 16;
  const int64_t row = min(n_base + r, N - 1);
  const uint8_t* pr = packed + row * (K >> 1);
  const uint8_t* sr = scales + row * (K >> 4);
  const int nchunks = (K + kChunk - 1) / kChunk;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();   // the previous chunk's fragment reads are done
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      const int v = tid + 256 * i;
      const int m = v >> 5, k = c * kChunk + 8 * (v & 31);
      const u32x4 val = *reinterpret_cast<const u32x4*>(x + (int64_t)min(m, M - 1) * K + min(k, K - 8));
      *reinterpret_cast<u32x4*>(&xs[m][8 * (v & 31)]) = (m < M && k < K) ? val : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int kb = c * kChunk + 64 * g;
    uint32_t pw[8], ws = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = kb + 16 * j;
      const int kc = min(kk, K - 16);
      const uint2 v = *reinterpret_cast<const uint2*>(pr + kc / 2);
      const uint32_t sbyte = sr[kc / 16];
      ws |= (kk < K ? sbyte : 0u) << (8 * j);
      pw[2 * j] = v.x;
      pw[2 * j + 1] = v.y;
    }
    const float sv[4] = {NVFP4_E4M3_TO_F32(ws, 0), NVFP4_E4M3_TO_F32(ws, 1), NVFP4_E4M3_TO_F32(ws, 2),
                         NVFP4_E4M3_TO_F32(ws, 3)};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 a = dequant8(pw[s], sv[s >> 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma16x16x32(a, *reinterpret_cast<const bf16x8*>(&xs[16 * mt + r][64 * g + 8 * s]), acc[mt]);
    }
  }
  if (n_base >= N) return;
  const float gs = *gs_ptr;
  const int n0 = n_base + 4 * g;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + r;
    if (m >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (n0 + v < N) y[(int64_t)m * N + n0 + v] = (uint16_t)out_bf16(acc[mt][v], gs, bias, n0 + v);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Workgroups of 256 threads that fit on the device at once (occupancy x CUs).
static int resident_workgroups(const void* kernel) {
  const int dev = current_device();
  return device_cus(dev) * blocks_per_cu(kernel, dev, 256, 0);
}

template <int MR, int SEG>
static hipError_t dot_launch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                             const float* gs, int N, const void* bias, void* y, hipStream_t stream) {
  // Batches of 4 rows dealt round-robin to the wavefronts: as many
  // wavefronts as fit at once, trimmed so that each takes the same number of
  // batches (within one).
  const void* fn = (const void*)gemv_dot_kernel<MR, SEG>;
  const int resident = 4 * resident_workgroups(fn);
  const int batches = (N + 3) / 4;
  const int per_wave = (batches + resident - 1) / resident;
  const int waves = (batches + per_wave - 1) / per_wave;
  return launch_kernel(fn, dim3((waves + 3) / 4), dim3(256), stream, (const uint16_t*)x, M, K, packed, scales, gs,
                       N, (const uint16_t*)bias, (uint16_t*)y, waves);
}

template <int MR>
static hipError_t dot_dispatch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                               const float* gs, int N, const void* bias, void* y, hipStream_t stream) {
  switch ((K + 2047) / 2048) {
    case 1: return dot_launch<MR, 1>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 2: return dot_launch<MR, 2>(x, M, K, packed, scales, gs, N, bias, y, stream);
    // two rows only reach here with K <= 4096 (decode_uses_dot)
    case 3: return dot_launch<1, 3>(x, M, K, packed, scales, gs, N, bias, y, stream);
    default: return dot_launch<1, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
  }
}

template <int MT, int R>
static hipError_t mfma_launch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                              const float* gs, int N, const void* bias, void* y, hipStream_t stream) {
  if (K % kChunk != 0)
    return launch_kernel((const void*)gemv_mfma_ragged_kernel<MT>, dim3((N + 63) / 64), dim3(256), stream,
                         (const uint16_t*)x, M, K, packed, scales, gs, N, (const uint16_t*)bias, (uint16_t*)y);
  const void* fn = (const void*)gemv_mfma_kernel<MT, R>;
  const int nblocks = (N + 64 * R - 1) / (64 * R);
  const dim3 grid(std::min(nblocks, resident_workgroups(fn)));
  return launch_kernel(fn, grid, dim3(256), stream, (const uint16_t*)x, M, K, packed, scales, gs, N,
                       (const uint16_t*)bias, (uint16_t*)y);
}

// The dot kernel keeps the lane's slice of x in registers (16 * ceil(K/2048)
// VGPRs per activation row), so it takes M = 1 up to K = 8192 and M = 2 up to
// K = 4096; everything else goes to the MFMA kernel.
// Dynamic LDS of gemv_xres_kernel<NW, false, 1, depth> for (M, K): x rows,
// NW per-wavefront weight (2 KiB per region: max(depth, 1) regions) and scale
// (1 KiB) regions, 16 row scales.
static int64_t xres_lds_bytes(int64_t M, int64_t K, int nw, int depth) {
  return M * (2 * K + 16) + (int64_t)nw * (2048 * (depth ? depth : 1) + 1024) + 16 * sizeof(float);
}

template <int NW, int kDepth>
static hipError_t xres_launch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                              const float* gs, int N, const void* bias, void* y, hipStream_t stream) {
  const void* fn = (const void*)gemv_xres_kernel<NW, false, 1, kDepth>;
  const int lds = (int)xres_lds_bytes(M, K, NW, kDepth);
  const int dev = current_device();
  const hipError_t e = ensure_dynamic_lds(fn, dev, kXresLdsMax);
  if (e != hipSuccess) return e;
  const int ntiles = (N + 15) / 16;
  const int resident = device_cus(dev) * blocks_per_cu(fn, dev, 64 * NW, lds);
  const int grid = std::max(1, std::min((ntiles + NW - 1) / NW, resident));
  return launch_kernel_lds(fn, dim3(grid), dim3(64 * NW), lds, stream, (const uint16_t*)x, M, K, packed, scales, gs,
                           N, (const uint16_t*)bias, (uint16_t*)y, MoeRows{nullptr, nullptr, 1, 0, 0, -1});
}

// Expert layer: gemv_xres_kernel<NW, true, KS> over a (G, E) grid for the
// experts with 1..mcap pairs (grid row E: the invalid ids' zero rows).  The
// plan picks, for 16 and for 8 wavefronts, the K split KS (2 or 4 keeping at
// least 8 chunks per wavefront, 8 keeping at least 4) that
// gives every wavefront slot of the GPU a tile when at most min(E, P)
// experts hold pairs, and the largest mcap (<= 16, <= P) whose activation
// rows fit in LDS next to the weight regions (and, for KS > 1, the partial
// tiles); the wider mcap wins, 16 wavefronts on a tie.  Without a K split
// (KS = 1) and with K % 1024 == 0, the two-region pipeline (depth 2) is used
// when the rows it can still hold cover twice the mean pair count of an
// active expert (its larger weight regions leave room for fewer activation
// rows; experts beyond mcap go to the panel kernel).  mcap = 0: none fits or
// K % 256 != 0.
static int64_t moe_xres_lds(int64_t m, int64_t K, int nw, int ks, int depth = 0) {
  return m * (2 * K + 16) + (int64_t)nw * (2048 * (depth ? depth : 1) + 1024) + 64 +
         (ks > 1 ? (int64_t)nw * 1024 : 0);
}

MoeXresPlan moe_xres_plan(int64_t P, int64_t E, int64_t K, int64_t N) {
  MoeXresPlan best{0, 0, 1, 0};
  if (K % kChunk != 0 || P < 1) return best;
  const int cus = device_cus(current_device());
  const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, P));
  const int64_t tiles = (N + 15) / 16 * active;
  const int64_t nchunks = K / kChunk;
  for (int nw : {16, 8}) {
    // split K while the tiles leave wavefront slots empty: in 2 or 4 while
    // each part keeps at least 8 chunks, in 8 (few active experts with long
    // rows, e.g. the down projection of one token) while it keeps 4
    int ks = 1;
    while (ks < 4 && tiles * ks < (int64_t)cus * nw && nchunks >= 8 * ks) ks *= 2;
    if (ks == 4 && tiles * ks < (int64_t)cus * nw && nchunks >= 32) ks = 8;
    int m = (int)std::min<int64_t>(16, P);
    while (m >= 1 && moe_xres_lds(m, K, nw, ks) > kXresLdsMax) --m;
    if (m > best.mcap) best = MoeXresPlan{m, nw, ks, 0};
  }
  if (best.ks == 1 && K % (4 * kChunk) == 0) {
    int m = best.mcap;
    while (m >= 1 && moe_xres_lds(m, K, best.nw, 1, 2) > kXresLdsMax) --m;
    const int64_t want = 2 * ((P + active - 1) / active);   // twice the mean pairs per active expert
    if (m >= std::min<int64_t>(best.mcap, want)) best = MoeXresPlan{m, best.nw, 1, 2};
  }
  return best;
}

template <int NW, int KS, int D = 0>
static hipError_t moe_xres_launch(const void* x, int row_div, int K, const int32_t* offsets, const int32_t* order,
                                  int mcap, int64_t P, const uint8_t* packed, const uint8_t* scales, const float* gs,
                                  int E, int N, void* y, hipStream_t stream) {
  const void* fn = (const void*)gemv_xres_kernel<NW, true, KS, D>;
  const int lds = (int)moe_xres_lds(mcap, K, NW, KS, D);
  const int dev = current_device();
  const hipError_t e = ensure_dynamic_lds(fn, dev, kXresLdsMax);
  if (e != hipSuccess) return e;
  const int cus = device_cus(dev), per_cu = blocks_per_cu(fn, dev, 64 * NW, lds);
  // at most min(E, P) experts have pairs: give each the workgroups that would
  // fill the GPU if all of them fell in this kernel's class, twice that when
  // the pairs average more than mcap / 2 per expert (then many experts have
  // more than mcap and belong to another kernel)
  const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, P));
  const int64_t fill = (2 * P > (int64_t)mcap * active ? 2 : 1) * (int64_t)cus * per_cu;
  const int ntiles = (N + 15) / 16, slots = NW / KS;
  const int64_t g = std::min<int64_t>((ntiles + slots - 1) / slots, (fill + active - 1) / active);
  const MoeRows moe{offsets, order, row_div, mcap, 1, E};   // row E of the grid: the invalid ids' zero rows
  return launch_kernel_lds(fn, dim3((unsigned)std::max<int64_t>(1, g), (unsigned)E + 1), dim3(64 * NW), lds, stream,
                           (const uint16_t*)x, 0, K, packed, scales, gs, N, (const uint16_t*)nullptr, (uint16_t*)y,
                           moe);
}

hipError_t launch_moe_xres(const void* x, int64_t row_div, int64_t K, const int32_t* offsets, const int32_t* order,
                           const MoeXresPlan& plan, int64_t P, const uint8_t* packed, const uint8_t* scales,
                           const float* gs, int64_t E, int64_t N, void* y, hipStream_t stream) {
  if (plan.mcap < 1) return hipSuccess;
#define NVFP4_MOE_XRES(NW_, KS_)                                                                              \
  return moe_xres_launch<NW_, KS_>(x, (int)row_div, (int)K, offsets, order, plan.mcap, P, packed, scales, gs, \
                                   (int)E, (int)N, y, stream)
  if (plan.depth == 2) {
    if (plan.nw == 16)
      return moe_xres_launch<16, 1, 2>(x, (int)row_div, (int)K, offsets, order, plan.mcap, P, packed, scales, gs,
                                       (int)E, (int)N, y, stream);
    return moe_xres_launch<8, 1, 2>(x, (int)row_div, (int)K, offsets, order, plan.mcap, P, packed, scales, gs,
                                    (int)E, (int)N, y, stream);
  }
  if (plan.nw == 16) {
    if (plan.ks == 8) NVFP4_MOE_XRES(16, 8);
    if (plan.ks == 4) NVFP4_MOE_XRES(16, 4);
    if (plan.ks == 2) NVFP4_MOE_XRES(16, 2);
    NVFP4_MOE_XRES(16, 1);
  }
  if (plan.ks == 8) NVFP4_MOE_XRES(8, 8);
  if (plan.ks == 4) NVFP4_MOE_XRES(8, 4);
  if (plan.ks == 2) NVFP4_MOE_XRES(8, 2);
  NVFP4_MOE_XRES(8, 1);
#undef NVFP4_MOE_XRES
}

// Panel width for gemv_panel_kernel: the widest multiple of 512 columns whose
// M rows fit in the x panel region.
static int panel_columns(int M, int K) {
  const int pk = (kPanelXBytes / M / 2) / 512 * 512;
  return std::min(pk, K);
}

template <int MT, int NW, int R>
static hipError_t panel_launch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                               const float* gs, int N, const void* bias, void* y, hipStream_t stream) {
  const void* fn = (const void*)gemv_panel_kernel<MT, NW, R>;
  const int nblocks = (N + 16 * NW * R - 1) / (16 * NW * R);
  const int dev = current_device();
  const dim3 grid(std::min(nblocks, device_cus(dev) * blocks_per_cu(fn, dev, 64 * NW, 0)));
  return launch_kernel(fn, grid, dim3(64 * NW), stream, (const uint16_t*)x, M, K, packed, scales, gs, N,
                       (const uint16_t*)bias, (uint16_t*)y, panel_columns(M, K), MoeRows{nullptr, nullptr, 1, 0, 0, -1});
}

// Expert layer: gemv_panel_kernel<MT, 8, R, true> over a (G, E) grid for the
// experts with mmin..mcap pairs (mcap <= 16 MT); K % 512 == 0.
template <int MT, int R>
static hipError_t moe_panel_launch(const void* x, int row_div, int K, const int32_t* offsets, const int32_t* order,
                                   int mmin, int mcap, int64_t P, const uint8_t* packed, const uint8_t* scales,
                                   const float* gs, int E, int N, void* y, bool zero_rows, hipStream_t stream) {
  const void* fn = (const void*)gemv_panel_kernel<MT, 8, R, true>;
  if (MT > 2) mcap = std::min(mcap, 16 * MT);          // the 64-row form runs one pass
  const int dev = current_device();
  const int cus = device_cus(dev), per_cu = blocks_per_cu(fn, dev, 64 * 8, 0);
  // at most P / mmin experts fall in the class: give each twice the workgroups
  // that would fill the GPU if all of them did
  const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, P / std::max(1, mmin)));
  const int nblocks = (N + 16 * 8 * R - 1) / (16 * 8 * R);
  const int64_t g = std::min<int64_t>(nblocks, (2 * cus * per_cu + active - 1) / active);
  // with zero_rows, grid row E writes the invalid ids' zero rows
  const MoeRows moe{offsets, order, row_div, mcap, mmin, zero_rows ? E : -1};
  return launch_kernel(fn, dim3((unsigned)std::max<int64_t>(1, g), (unsigned)E + (zero_rows ? 1 : 0)), dim3(64 * 8),
                       stream,
                       (const uint16_t*)x, 0, K, packed, scales, gs, N, (const uint16_t*)nullptr, (uint16_t*)y,
                       panel_columns(std::min(mcap, 16 * MT), K), moe);
}

hipError_t launch_moe_panel(const void* x, int64_t row_div, int64_t K, const int32_t* offsets, const int32_t* order,
                            int mmin, int mcap, int rows, int64_t P, const uint8_t* packed, const uint8_t* scales,
                            const float* gs, int64_t E, int64_t N, void* y, bool zero_rows, hipStream_t stream) {
  if (mmin > mcap || K % 512 != 0) return hipSuccess;
  // 512 rows per workgroup (4 tiles per wavefront) when the expert has enough
  // rows to fill the GPU with such blocks, else 128 (one tile per wavefront)
  const bool wide = N >= 16384;
#define NVFP4_MOE_PANEL(MT_)                                                                                     \
  (wide ? moe_panel_launch<MT_, 4>(x, (int)row_div, (int)K, offsets, order, mmin, mcap, P, packed, scales, gs,   \
                                   (int)E, (int)N, y, zero_rows, stream)                                        \
        : moe_panel_launch<MT_, 1>(x, (int)row_div, (int)K, offsets, order, mmin, mcap, P, packed, scales, gs,   \
                                   (int)E, (int)N, y, zero_rows, stream))
  if (rows <= 16) return NVFP4_MOE_PANEL(1);
  if (rows <= 32) return NVFP4_MOE_PANEL(2);
  return NVFP4_MOE_PANEL(4);
#undef NVFP4_MOE_PANEL
}

// Dynamic LDS of gemv_xphase_kernel<NW, TW> for M rows and phases of kp
// columns: x rows, two weight regions and a scale region per wavefront, 16
// row scales.
static int64_t xphase_lds_bytes(int64_t M, int64_t kp, int nw, int depth) {
  return M * (2 * kp + 16) + (int64_t)nw * (depth * 2048 + 1024) + 16 * sizeof(float);
}

// Phase width for the phased x-resident kernel (16 wavefronts, two regions
// each): K / 2, K / 4 or K / 8, the widest whose x rows fit in LDS beside the
// regions and that is a multiple of 1024 columns, or 0.  Measured against
// the panel kernel (random codes, one box): 8B shape M = 16 55.7 against
// 61.4 us; 70B shape M = 8 / 12 / 16 120.5 / 117.4 / 118.2 against 126.0 /
// 121.4 / 120.9 us.  Eight wavefronts (two or three regions) and sixteen
// with three regions were slower or no faster.
constexpr int kXphaseNW = 16, kXphaseDepth = 2;
static int64_t xphase_kp(int64_t M, int64_t K) {
  if (M < 3 || M > 16) return 0;
  for (int64_t np = 2; np <= 8; np *= 2)
    if (K % np == 0 && (K / np) % 1024 == 0 && xphase_lds_bytes(M, K / np, kXphaseNW, kXphaseDepth) <= kXresLdsMax)
      return K / np;
  return 0;
}

template <int NW, int TW, int D>
static hipError_t xphase_launch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                                const float* gs, int N, const void* bias, void* y, int kp, int grid,
                                hipStream_t stream) {
  const void* fn = (const void*)gemv_xphase_kernel<NW, TW, D>;
  const hipError_t e = ensure_dynamic_lds(fn, current_device(), kXresLdsMax);
  if (e != hipSuccess) return e;
  return launch_kernel_lds(fn, dim3(grid), dim3(64 * NW), (size_t)xphase_lds_bytes(M, kp, NW, D), stream,
                           (const uint16_t*)x, M, K, packed, scales, gs, N, (const uint16_t*)bias, (uint16_t*)y, kp);
}

// One workgroup per resident slot (at most one per NW tiles), each
// wavefront taking up to TW = 1, 2 or 4 tiles; `grid` and `tw` give the
// plan, or tw = 0 when more than 4 tiles per wavefront would be needed
// (N > 262144 on 256 compute units: left to the panel kernel).
static void xphase_plan(int M, int kp, int N, int* grid, int* tw) {
  const int dev = current_device();
  const void* fn = (const void*)gemv_xphase_kernel<kXphaseNW, 4, kXphaseDepth>;   // every TW takes the same LDS
  const int ntiles = (N + 15) / 16;
  const int resident = device_cus(dev) *
                       blocks_per_cu(fn, dev, 64 * kXphaseNW, (size_t)xphase_lds_bytes(M, kp, kXphaseNW, kXphaseDepth));
  *grid = std::max(1, std::min((ntiles + kXphaseNW - 1) / kXphaseNW, resident));
  *tw = (ntiles + *grid * kXphaseNW - 1) / (*grid * kXphaseNW);
  if (*tw > 4) *tw = 0;
}

static hipError_t xphase_dispatch(const void* x, int M, int K, const uint8_t* packed, const uint8_t* scales,
                                  const float* gs, int N, const void* bias, void* y, int kp, int grid, int tw,
                                  hipStream_t stream) {
  constexpr int NW = kXphaseNW, D = kXphaseDepth;
  if (tw <= 1) return xphase_launch<NW, 1, D>(x, M, K, packed, scales, gs, N, bias, y, kp, grid, stream);
  if (tw <= 2) return xphase_launch<NW, 2, D>(x, M, K, packed, scales, gs, N, bias, y, kp, grid, stream);
  return xphase_launch<NW, 4, D>(x, M, K, packed, scales, gs, N, bias, y, kp, grid, stream);
}

// x-resident configuration for (M, K): 10 * wavefronts + pipeline depth (2
// or 3 regions, K % 1024 == 0; 0 for the single-region form), or 0 to leave
// (M, K) to the streaming kernels.  Measured on the 8B shape (K = 4096): 8
// wavefronts with two regions are fastest up to M = 8 (three regions are no
// faster), 16 beyond; when only 8 single-region wavefronts fit and K %
// 1024 == 0, the panel kernel is faster (M = 16: 58-60 vs 67 us).
static int xres_config(int64_t M, int64_t K) {
  if (M < 3 || M > 16 || K % kChunk != 0) return 0;
  const bool deep = K % (4 * kChunk) == 0;
  static constexpr int kSmall[][2] = {{8, 2}, {16, 2}, {16, 0}};
  static constexpr int kLarge[][2] = {{16, 2}, {16, 0}, {8, 2}};
  for (const auto& c : (M <= 8 ? kSmall : kLarge))
    if ((c[1] == 0 || deep) && xres_lds_bytes(M, K, c[0], c[1]) <= kXresLdsMax) return 10 * c[0] + c[1];
  if (!deep && xres_lds_bytes(M, K, 8, 0) <= kXresLdsMax) return 80;
  return 0;
}

bool decode_uses_dot(int64_t M, int64_t K) {
  return K % 32 == 0 && ((M == 1 && K <= 8192) || (M == 2 && K <= 4096));
}

hipError_t launch_gemv(const void* x, int64_t M64, int64_t K64, const uint8_t* packed, const uint8_t* scales,
                       const float* gs, int64_t N64, const void* bias, void* y, hipStream_t stream) {
  const int M = (int)M64, K = (int)K64, N = (int)N64;
  if (decode_uses_dot(M, K)) {
    if (M == 1) return dot_dispatch<1>(x, M, K, packed, scales, gs, N, bias, y, stream);
    return dot_dispatch<2>(x, M, K, packed, scales, gs, N, bias, y, stream);
  }
  switch (xres_config(M, K)) {
    case 82: return xres_launch<8, 2>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 162: return xres_launch<16, 2>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 160: return xres_launch<16, 0>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 80: return xres_launch<8, 0>(x, M, K, packed, scales, gs, N, bias, y, stream);
    default: break;
  }
  if (const int64_t kp = xphase_kp(M, K)) {
    int grid = 0, tw = 0;
    xphase_plan(M, (int)kp, N, &grid, &tw);
    if (tw > 0) return xphase_dispatch(x, M, K, packed, scales, gs, N, bias, y, (int)kp, grid, tw, stream);
  }
  if (K % 512 == 0) {
    switch ((M + 15) / 16) {
      case 1: return panel_launch<1, 8, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
      case 2: return panel_launch<2, 8, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
      case 3: return panel_launch<3, 8, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
      default: return panel_launch<4, 8, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
    }
  }
  switch ((M + 15) / 16) {
    case 1: return mfma_launch<1, 1>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 2: return mfma_launch<2, 2>(x, M, K, packed, scales, gs, N, bias, y, stream);
    case 3: return mfma_launch<3, 2>(x, M, K, packed, scales, gs, N, bias, y, stream);
    default: return mfma_launch<4, 4>(x, M, K, packed, scales, gs, N, bias, y, stream);
  }
}

}  // namespace nvfp4
