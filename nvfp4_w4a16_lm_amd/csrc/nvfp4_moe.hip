// NVFP4 W4A16 mixture-of-experts layer for gfx950: per-expert NVFP4 weights,
// bf16 activations, top-k routing.
//
// Method: vLLM modelopt.py, ModelOptNvFp4FusedMoE (use_a16: weight-only NVFP4
// experts; w13 [E, 2I, H/2] with e4m3 scales [E, 2I, H/16] and one global
// scale per expert, the w1 column of w13_weight_scale_2; w2 [E, H, I/2] with
// scales [E, H, I/16] and global scales [E]; apply() takes the activations,
// topk_weights and topk_ids).  The NVFP4 format and its dequantization are
// those of the lm_head path (vLLM API docs, quantization.online.lm_head).
//
// Pair p = t * topk + j is token t's j-th routed expert topk_ids[t, j].
//
// moe_route_kernel: one workgroup groups the pairs by expert, in increasing
//   pair order inside each expert (a stable counting sort: threads own
//   (expert, segment) cells, count, prefix-sum the cells in order, then
//   scatter).  Pairs whose id is outside [0, E) form an extra group E.
// Experts with 1..mcap pairs (mcap <= 16: as many activation rows as fit in
//   LDS; none when, with K % 512 == 0, the pairs average more than mcap / 2
//   per active expert, so that one panel launch covers them all) run the
//   lm_head path's x-resident decode kernel (gemv_xres_kernel in
//   nvfp4_decode.hip, over a (workgroups, E) grid with the expert's gathered
//   rows converted to f16 in LDS and weights copied straight to LDS; when the
//   active experts have few 16-row tiles it splits each tile's K over 2, 4
//   or 8 wavefronts).  Its grid has a row E more, which writes the zero rows
//   of pairs whose id is outside [0, E).
// With K % 512 == 0, experts with more pairs, up to 64, run the lm_head
//   path's panel decode kernel (gemv_panel_kernel, same row gathering); when
//   the pairs average at most 16 per active expert, one launch of its 32-row
//   form takes every such expert, one with more than 32 pairs in passes of
//   32 rows over its weights.
// moe_gemv_kernel (otherwise, the other experts with at most 48 pairs): a
//   workgroup of 4 wavefronts owns 32 to 128 weight rows of one expert and
//   splits K between 1, 2 or 4 of its wavefronts; each streams its weights
//   and scales straight into registers one 256-k chunk ahead (two alternating
//   buffers) and its activation fragments per chunk, with no barrier,
//   dequantizes exactly (code * scale is a bf16 value) and runs bf16 MFMA
//   (v_mfma_f32_16x16x32_bf16, 16 pairs per column tile); the partial tiles
//   are summed through LDS in wavefront order.  When the x-resident kernel
//   does not run (K % 256 != 0, or no activation row fits in LDS), it writes
//   the zero rows of pairs whose id is outside [0, E).
// moe_gemm_kernel (experts with more than 64 pairs, or 48 when K % 512 !=
//   0): a workgroup of 4 wavefronts streams 256 weight rows of one expert
//   once per block of 64 pairs; each wavefront owns 4 tiles of 16 rows, loads
//   its weights straight into registers one chunk ahead and runs the same
//   MFMA against the gathered activation rows staged in LDS.
// In the last two, the k order inside a chunk is permuted identically on both
// operands so that a lane's codes are two 16-byte loads.
// moe_silu_mul_kernel: a = silu(h[:, :I]) * h[:, I:] in float32, one bf16
//   rounding.
// moe_combine_kernel: out[t] = sum_j w[t, j] * o[t * topk + j] in float32 in
//   slot order, one bf16 rounding.
#include <algorithm>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kMoeThreads = 256;     // 4 wavefronts
constexpr int kMoeRows = 256;        // weight rows per workgroup (4 wavefronts x 4 tiles x 16)
constexpr int kMoeMBlock = 64;       // pairs per block (4 MFMA column tiles)
constexpr int kMoeChunk = 256;       // k per chunk
constexpr int kRouteThreads = 1024;
constexpr int kMoeSmallMax = 48;     // experts with at most this many pairs take moe_gemv_kernel
constexpr int kGemvWaves = 4;        // moe_gemv_kernel: wavefronts splitting K
constexpr int kGemvTiles = 2;        // moe_gemv_kernel: 16-row tiles per workgroup

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// Routing.  Workspace (int32): offsets[E + 2] (group g holds order[offsets[g]
// .. offsets[g + 1]); group E = invalid ids), then order[P].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ order,
                                                                  uint32_t* __restrict__ invalid_out) {
  __shared__ int32_t cell[kRouteThreads + 1];
  const int tid = threadIdx.x;
  const int groups = E + 1;
  // cells: S segments per group when groups <= 1024, else one cell per group
  // walked by thread g % 1024 (cells of one thread counted in group order)
  const int S = groups <= kRouteThreads ? max(1, kRouteThreads / groups) : 1;
  const int seg = (P + S - 1) / S;
  auto group_of = [&](int p) {
    const int v = ids[p];
    return (v < 0 || v >= E) ? E : v;
  };
  if (groups <= kRouteThreads) {
    __shared__ int32_t wave_sum[kRouteThreads / 64];
    const int g = tid / S, s = tid - g * S;
    const int lane = tid & 63, wave = tid >> 6;
    int c = 0;
    const int p0 = s * seg, p1 = min(P, p0 + seg);
    if (g < groups)
      for (int p = p0; p < p1; ++p) c += group_of(p) == g;
    // exclusive prefix of the cells in (group, segment) order = thread order:
    // wavefront scans, then a scan of the 16 wavefront totals
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) wave_sum[wave] = v;
    __syncthreads();
    if (wave == 0) {
      int w = lane < kRouteThreads / 64 ? wave_sum[lane] : 0;
#pragma unroll
      for (int off = 1; off < kRouteThreads / 64; off <<= 1) {
        const int t = __shfl_up(w, off, 64);
        if (lane >= off) w += t;
      }
      if (lane < kRouteThreads / 64) wave_sum[lane] = w;
    }
    __syncthreads();
    const int incl = v + (wave > 0 ? wave_sum[wave - 1] : 0);
    const int excl = incl - c;
    const int total = wave_sum[kRouteThreads / 64 - 1];
    if (g < groups && s == 0) offsets[g] = excl;
    if (tid == 0) offsets[groups] = total;
    if (g == E && s == 0 && invalid_out) *invalid_out = (uint32_t)(total - excl);
    if (g < groups) {
      int at = excl;
      for (int p = p0; p < p1; ++p)
        if (group_of(p) == g) order[at++] = p;
    }
  } else {
    // many experts: thread t owns groups t, t + 1024, ...; count, prefix per
    // thread in group order, then one more serial pass per group
    __shared__ int32_t base;
    if (tid == 0) base = 0;
    __syncthreads();
    for (int g0 = 0; g0 < groups; g0 += kRouteThreads) {
      const int g = g0 + tid;
      int c = 0;
      if (g < groups)
        for (int p = 0; p < P; ++p) c += group_of(p) == g;
      cell[tid] = c;
      __syncthreads();
      if (tid == 0) {
        int run = base;
        for (int i = 0; i < kRouteThreads && g0 + i < groups; ++i) {
          const int v = cell[i];
          cell[i] = run;
          offsets[g0 + i] = run;
          run += v;
        }
        base = run;
      }
      __syncthreads();
      if (g < groups) {
        int at = cell[tid];
        for (int p = 0; p < P; ++p)
          if (group_of(p) == g) order[at++] = p;
      }
      __syncthreads();
    }
    if (tid == 0) {
      offsets[groups] = base;
      if (invalid_out) *invalid_out = (uint32_t)(base - offsets[E]);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM: y[p, n] = bf16(gs_e * sum_k x[p / row_div, k] * deq(W_e)[n, k])
// for every pair p of expert e; rows of invalid pairs are zero.
//
// Chunk layout (256 k): lane (r, g) = (lane % 16, lane / 16) loads, for its
// row, code bytes [64 j + 16 g, +16) (j = 0, 1), i.e. k = 128 j + 32 g + [0, 32);
// MFMA step s (0..7) uses k = 128 (s / 4) + 32 g + 8 (s % 4) + [0, 8), whose
// block is 8 (s / 4) + 2 g + (s % 4) / 2.  The activation tile is stored in
// LDS as 64 rows x 32 pieces of 16 bytes (8 k), piece q of row m at slot
// q ^ (m & 15); step s of lane g reads piece 16 (s / 4) + 4 g + s % 4.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(const uint16_t* __restrict__ x, int row_div, int K,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ order,
                                                               const uint8_t* __restrict__ packed,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ gs_arr, int N,
                                                               uint16_t* __restrict__ y, int large_min) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kMoeMBlock * kMoeChunk * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;
  const int first = offsets[e], cnt = offsets[e + 1] - first;
  if (cnt <= large_min) return;                       // another kernel's (uniform over the workgroup)
  const int nb = blockIdx.x * kMoeRows;
  const int64_t prow = K >> 1, srow = K >> 4;
  const uint8_t* const wbase = packed + (int64_t)e * N * prow;
  const uint8_t* const sbase = scales + (int64_t)e * N * srow;
  const float gs = gs_arr[e];
  const int nchunks = (K + kMoeChunk - 1) / kMoeChunk;
  const int nw = nb + 64 * wave;                      // this wavefront's first row
  int64_t wrow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) wrow[t] = min(nw + 16 * t + r, N - 1);

  // this lane's weight words (two 16-byte pieces) and 4 scale bytes of tile t, chunk c
  auto load_w = [&](int t, int c, u32x4* w, uint32_t* sc) {
    const uint8_t* row = wbase + wrow[t] * prow;
    const uint8_t* srw = sbase + wrow[t] * srow;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k0 = kMoeChunk * c + 128 * j + 32 * g;        // first k of the piece
      if (k0 + 32 <= K) {
        if ((K & 31) == 0) {                                  // rows are 16-byte aligned
          w[j] = load_stream16(row + (k0 >> 1));
        } else {
          const uint2 h0 = *reinterpret_cast<const uint2*>(row + (k0 >> 1));
          const uint2 h1 = *reinterpret_cast<const uint2*>(row + (k0 >> 1) + 8);
          w[j] = u32x4{h0.x, h0.y, h1.x, h1.y};
        }
      } else if (k0 < K) {                                    // K % 32 == 16: 16 codes
        const uint2 h = *reinterpret_cast<const uint2*>(row + (k0 >> 1));
        w[j] = u32x4{h.x, h.y, 0u, 0u};
      } else {
        w[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 16 * c + 8 * j + 2 * g + h;             // block index in the row
        if (b < (K >> 4)) s |= (uint32_t)srw[b] << (8 * (2 * j + h));
      }
    }
    *sc = s;
  };

  for (int mb = 0; mb < cnt; mb += kMoeMBlock) {
    const int mrows = min(kMoeMBlock, cnt - mb);
    const int mtiles = (mrows + 15) / 16;
    // x staging: this thread's pieces of the block's rows (row m, piece q)
    auto load_x = [&](int c, u32x4* xv) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + kMoeThreads * i, m = id >> 5, q = id & 31;
        const int k0 = kMoeChunk * c + 8 * q;
        if (m < 16 * mtiles && k0 < K) {
          const int src = order[first + mb + min(m, mrows - 1)] / row_div;
          xv[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)src * K + k0);
        } else {
          xv[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_x = [&](const u32x4* xv) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + kMoeThreads * i, m = id >> 5, q = id & 31;
        if (m < 16 * mtiles) *reinterpret_cast<u32x4*>(xs + 512 * m + 16 * (q ^ (m & 15))) = xv[i];
      }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wcur[4][2], wnext[4][2];
    uint32_t scur[4], snext[4];
    u32x4 xv[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) load_w(t, 0, wcur[t], &scur[t]);
    load_x(0, xv);
    __syncthreads();                                  // the previous block's reads of xs are done
    store_x(xv);
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
      const bool more = c + 1 < nchunks;
      if (more) {
#pragma unroll
        for (int t = 0; t < 4; ++t) load_w(t, c + 1, wnext[t], &snext[t]);
        load_x(c + 1, xv);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 bx[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mt < mtiles) {
            const int m = 16 * mt + r;
            const int q = 16 * (s >> 2) + 4 * g + (s & 3);
            bx[mt] = *reinterpret_cast<const bf16x8*>(xs + 512 * m + 16 * (q ^ (m & 15)));
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t sb = (scur[t] >> (8 * (2 * (s >> 2) + ((s & 3) >> 1)))) & 0xFFu;
          const bf16x8 a = dequant8(wcur[t][s >> 2][s & 3], NVFP4_E4M3_TO_F32(sb, 0));
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            if (mt < mtiles) acc[t][mt] = mfma_bf16(a, bx[mt], acc[t][mt]);
        }
      }
      if (more) {
        __syncthreads();                              // every wavefront is done with chunk c
        store_x(xv);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wcur[t][0] = wnext[t][0];
          wcur[t][1] = wnext[t][1];
          scur[t] = snext[t];
        }
        __syncthreads();
      }
    }

    // epilogue: lane holds weight rows 16 t + 4 g + v, block row 16 mt + r
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = 16 * mt + r;
      if (mt >= mtiles || m >= mrows) continue;
      uint16_t* yrow = y + (int64_t)order[first + mb + m] * N;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n0 = nw + 16 * t + 4 * g;
        if ((N & 3) == 0 && n0 + 3 < N) {
          const uint32_t lo = f32_to_bf16_rne(acc[t][mt][0] * gs) | (f32_to_bf16_rne(acc[t][mt][1] * gs) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc[t][mt][2] * gs) | (f32_to_bf16_rne(acc[t][mt][3] * gs) << 16);
          *reinterpret_cast<uint2*>(yrow + n0) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n0 + v < N) yrow[n0 + v] = (uint16_t)f32_to_bf16_rne(acc[t][mt][v] * gs);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM for experts with at most kMoeSmallMax pairs (decode-sized
// routing).  A workgroup of 4 wavefronts owns 16 R rows of one expert per
// row group; K is split over `splitk` wavefronts of a group (wavefront w takes
// chunks w % splitk, + splitk, ...; splitk = 1, 2 or 4 so that each streams at
// least 8 chunks when K allows), each loading
// its weights and scales straight into registers one chunk ahead and the
// chunk's activation fragments (small, L2-resident) as it starts it, with no
// barrier until the end, where the partial tiles of a row group are
// summed through LDS in wavefront order.  Pairs are taken 16 at a time (one
// MFMA column tile); the activation fragments use the chunk layout of
// moe_gemm_kernel.  Group E (ids outside [0, E)) writes zero rows here.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(64 * kGemvWaves) void moe_gemv_kernel(const uint16_t* __restrict__ x, int row_div,
                                                                   int K, const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ order,
                                                                   const uint8_t* __restrict__ packed,
                                                                   const uint8_t* __restrict__ scales,
                                                                   const float* __restrict__ gs_arr, int E, int N,
                                                                   uint16_t* __restrict__ y, int splitk,
                                                                   int small_min) {
  __shared__ float red[kGemvWaves][4 * R][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;
  const int first = offsets[e], cnt = offsets[e + 1] - first;
  if (cnt == 0) return;                               // uniform over the workgroup
  // wavefront w: row group w / splitk (16 R rows), chunks w % splitk + j * splitk
  const int wg_rows = 16 * R * (kGemvWaves / splitk);
  const int nb = blockIdx.x * wg_rows;
  const int rg = wave / splitk, ph = wave - rg * splitk;
  if (e == E) {                                       // invalid ids: zero rows, this block's columns
    const int cols = min(wg_rows, N - nb);
    for (int i = tid; i < cnt * cols; i += 64 * kGemvWaves) {
      const int q = i / cols, c = i - q * cols;
      y[(int64_t)order[first + q] * N + nb + c] = 0;
    }
    return;
  }
  if (cnt <= small_min || cnt > kMoeSmallMax) return; // the x-resident kernel's or moe_gemm_kernel's
  const int64_t prow = K >> 1, srow = K >> 4;
  const uint8_t* const wbase = packed + (int64_t)e * N * prow;
  const uint8_t* const sbase = scales + (int64_t)e * N * srow;
  const float gs = gs_arr[e];
  const int nchunks = (K + kMoeChunk - 1) / kMoeChunk;
  const uint8_t* wrowp[R];
  const uint8_t* srowp[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int64_t row = min(nb + 16 * R * rg + 16 * t + r, N - 1);
    wrowp[t] = wbase + row * prow;
    srowp[t] = sbase + row * srow;
  }

  struct Chunk {
    u32x4 w[R][2];
    uint32_t sc[R];
  };
  auto load = [&](int c, Chunk& ch) {
#pragma unroll
    for (int t = 0; t < R; ++t) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k0 = kMoeChunk * c + 128 * j + 32 * g;
        if (k0 + 32 <= K) {
          if ((K & 31) == 0) {
            ch.w[t][j] = load_stream16(wrowp[t] + (k0 >> 1));
          } else {
            const uint2 h0 = *reinterpret_cast<const uint2*>(wrowp[t] + (k0 >> 1));
            const uint2 h1 = *reinterpret_cast<const uint2*>(wrowp[t] + (k0 >> 1) + 8);
            ch.w[t][j] = u32x4{h0.x, h0.y, h1.x, h1.y};
          }
        } else if (k0 < K) {
          const uint2 h = *reinterpret_cast<const uint2*>(wrowp[t] + (k0 >> 1));
          ch.w[t][j] = u32x4{h.x, h.y, 0u, 0u};
        } else {
          ch.w[t][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      uint32_t sv = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int b = 16 * c + 8 * j + 2 * g + h;
          if (b < (K >> 4)) sv |= (uint32_t)srowp[t][b] << (8 * (2 * j + h));
        }
      ch.sc[t] = sv;
    }
  };

  for (int mb = 0; mb < cnt; mb += 16) {
    const int mrows = min(16, cnt - mb);
    const uint16_t* const xr = x + (int64_t)(order[first + mb + min(r, mrows - 1)] / row_div) * K;
    f32x4 acc[R];
#pragma unroll
    for (int t = 0; t < R; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // chunk c of this wavefront: its activation fragments are loaded first
    // (L2-resident), then the weights of the wavefront's next chunk are issued
    // into the other buffer, then chunk c computes; the two weight buffers
    // alternate without register copies (a copy would wait for the loads), so
    // the prefetch stays in flight while the MFMAs run
    auto step = [&](int c, const Chunk& ch, Chunk& refill) {
      u32x4 xv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int k0 = kMoeChunk * c + 128 * (s >> 2) + 32 * g + 8 * (s & 3);
        xv[s] = k0 < K ? *reinterpret_cast<const u32x4*>(xr + k0) : u32x4{0u, 0u, 0u, 0u};
      }
      if (c + splitk < nchunks) load(c + splitk, refill);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 bx = __builtin_bit_cast(bf16x8, xv[s]);
#pragma unroll
        for (int t = 0; t < R; ++t) {
          const uint32_t sb = (ch.sc[t] >> (8 * (2 * (s >> 2) + ((s & 3) >> 1)))) & 0xFFu;
          acc[t] = mfma_bf16(dequant8(ch.w[t][s >> 2][s & 3], NVFP4_E4M3_TO_F32(sb, 0)), bx, acc[t]);
        }
      }
    };
    Chunk ca, cb;
    if (ph < nchunks) load(ph, ca);
    for (int c = ph; c < nchunks; c += 2 * splitk) {
      step(c, ca, cb);
      if (c + splitk >= nchunks) break;
      step(c + splitk, cb, ca);
    }
    // partial tiles -> LDS; lane (r, g) of tile t holds rows 16 t + 4 g + v, pair r
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][4 * t + v][lane] = acc[t][v];
    __syncthreads();
    for (int i = tid; i < 16 * wg_rows; i += 64 * kGemvWaves) {
      const int m = i / wg_rows, nl = i - m * wg_rows;
      const int g_of = nl / (16 * R), nl2 = nl - g_of * (16 * R);
      const int t = nl2 >> 4, gg = (nl2 >> 2) & 3, v = nl2 & 3;
      const int n = nb + nl;
      float sum = 0.f;
      for (int q = 0; q < splitk; ++q) sum += red[g_of * splitk + q][4 * t + v][16 * gg + m];
      if (m < mrows && n < N) y[(int64_t)order[first + mb + m] * N + n] = (uint16_t)f32_to_bf16_rne(sum * gs);
    }
    __syncthreads();                                  // red is reused by the next 16 pairs
  }
}

// ---------------------------------------------------------------------------
// a[p, i] = bf16(silu(h[p, i]) * h[p, I + i]); 8 outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_silu_mul_kernel(const uint16_t* __restrict__ h, int64_t P, int I,
                                                           uint16_t* __restrict__ a) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-wide vector index
  const int per_row = I / 8;
  if (v >= P * per_row) return;
  const int64_t p = v / per_row;
  const int i0 = (int)(v - p * per_row) * 8;
  const u32x4 gv = *reinterpret_cast<const u32x4*>(h + p * 2 * I + i0);
  const u32x4 uv = *reinterpret_cast<const u32x4*>(h + p * 2 * I + I + i0);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float g0 = bf16_lo(gv[e]), g1 = bf16_hi(gv[e]);
    const float s0 = g0 / (1.0f + expf(-g0)), s1 = g1 / (1.0f + expf(-g1));
    o[e] = f32_to_bf16_rne(s0 * bf16_lo(uv[e])) | (f32_to_bf16_rne(s1 * bf16_hi(uv[e])) << 16);
  }
  *reinterpret_cast<u32x4*>(a + p * I + i0) = o;
}

// ---------------------------------------------------------------------------
// out[t, n] = bf16(sum_j w[t, j] * o[t * topk + j, n]); 8 outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ o,
                                                          const float* __restrict__ w, int64_t T, int topk,
                                                          int H, uint16_t* __restrict__ out) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = H / 8;
  if (v >= T * per_row) return;
  const int64_t t = v / per_row;
  const int n0 = (int)(v - t * per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const float wj = w[t * topk + j];
    const u32x4 ov = *reinterpret_cast<const u32x4*>(o + (t * topk + j) * H + n0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __builtin_fmaf(wj, bf16_lo(ov[e]), acc[2 * e]);
      acc[2 * e + 1] = __builtin_fmaf(wj, bf16_hi(ov[e]), acc[2 * e + 1]);
    }
  }
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = f32_to_bf16_rne(acc[2 * e]) | (f32_to_bf16_rne(acc[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + t * H + n0) = r;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_moe_route(const int32_t* ids, int64_t P, int64_t E, int32_t* route_ws, uint32_t* invalid,
                            hipStream_t stream) {
  int32_t* offsets = route_ws;
  int32_t* order = route_ws + moe_route_offsets_words(E);
  return launch_kernel((const void*)moe_route_kernel, dim3(1), dim3(kRouteThreads), stream, ids, (int)P, (int)E,
                       offsets, order, invalid);
}

hipError_t launch_moe_gemm(const void* x, int64_t row_div, int64_t K, const int32_t* route_ws, int64_t P,
                           const uint8_t* packed, const uint8_t* scales, const float* gs, int64_t E, int64_t N,
                           void* y, hipStream_t stream) {
  const int32_t* offsets = route_ws;
  const int32_t* order = route_ws + moe_route_offsets_words(E);
  // experts with 1..mcap pairs: the x-resident decode kernel; with K % 512 == 0
  // the panel decode kernel takes the rest (up to 64 pairs, or all of them
  // in passes of 32 at <= 16 pairs per active expert), else the split-K
  // kernel up to 48; moe_gemm_kernel takes larger experts
  MoeXresPlan plan = moe_xres_plan(P, E, K, N);
  {
    // when the pairs average more than mcap / 2 per active expert, most
    // experts exceed mcap and the x-resident kernel would run only the few
    // left: the panel kernel then takes every expert, one launch over all of
    // them (moe_8x4096, 16 tokens: down projection 136 -> ~80 us)
    const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, P));
    if (K % 512 == 0 && 2 * P > (int64_t)plan.mcap * active) plan.mcap = 0;
  }
  const int mcap = plan.mcap;
  hipError_t err = launch_moe_xres(x, row_div, K, offsets, order, plan, P, packed, scales, gs, E, N, y, stream);
  if (err != hipSuccess) return err;
  bool zero_done = mcap >= 1;                         // the x-resident kernel writes the invalid ids' zero rows
  int small_min = mcap, large_min = kMoeSmallMax;
  if (K % 512 == 0) {
    const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, P));
    if (P > mcap && P <= 16 * active) {
      // at most 16 pairs per active expert on average: one launch of the
      // 32-row panel kernel takes every expert beyond mcap, the rare one
      // with more than 32 pairs in several passes, instead of two more
      // launches that would mostly find no expert in their class
      err = launch_moe_panel(x, row_div, K, offsets, order, mcap + 1, INT32_MAX, 32, P, packed, scales, gs, E, N, y,
                             !zero_done, stream);
      zero_done = true;
      large_min = INT32_MAX;
    } else {
      if (P > mcap) {                                 // else the first panel kernel writes them
        err = launch_moe_panel(x, row_div, K, offsets, order, mcap + 1, 32, 32, P, packed, scales, gs, E, N, y,
                               !zero_done, stream);
        zero_done = true;
      }
      if (err == hipSuccess && P > 32)
        err = launch_moe_panel(x, row_div, K, offsets, order, std::max(mcap + 1, 33), 64, 64, P, packed, scales, gs,
                               E, N, y, false, stream);
      large_min = 64;
    }
    if (err != hipSuccess) return err;
    small_min = kMoeSmallMax;                         // no expert left for the split-K kernel
  }
  // the split-K kernel takes experts with small_min < pairs <= 48 and writes
  // the invalid ids' zero rows; it is launched only if an expert can fall in
  // its class or no other kernel writes those rows
  if (!zero_done || (small_min < kMoeSmallMax && P > small_min)) {
    // K split over 1, 2 or 4 wavefronts so that each streams at least 8 chunks
    const int64_t nchunks = (K + kMoeChunk - 1) / kMoeChunk;
    const int splitk = nchunks >= 32 ? 4 : nchunks >= 16 ? 2 : 1;
    const int64_t wg_rows = 16 * kGemvTiles * (kGemvWaves / splitk);
    const dim3 grid_small((unsigned)((N + wg_rows - 1) / wg_rows), (unsigned)(E + 1));
    err = launch_kernel((const void*)moe_gemv_kernel<kGemvTiles>, grid_small, dim3(64 * kGemvWaves), stream,
                        reinterpret_cast<const uint16_t*>(x), (int)row_div, (int)K, offsets, order, packed, scales,
                        gs, (int)E, (int)N, reinterpret_cast<uint16_t*>(y), splitk, small_min);
  }
  if (err != hipSuccess || P <= large_min) return err;   // no expert can have more pairs
  const dim3 grid((unsigned)((N + kMoeRows - 1) / kMoeRows), (unsigned)E);
  return launch_kernel((const void*)moe_gemm_kernel, grid, dim3(kMoeThreads), stream,
                       reinterpret_cast<const uint16_t*>(x), (int)row_div, (int)K, offsets, order, packed, scales,
                       gs, (int)N, reinterpret_cast<uint16_t*>(y), large_min);
}

hipError_t launch_moe_silu_mul(const void* h, int64_t P, int64_t I, void* a, hipStream_t stream) {
  const int64_t vecs = P * I / 8;
  return launch_kernel((const void*)moe_silu_mul_kernel, dim3((unsigned)std::max<int64_t>(1, (vecs + 255) / 256)),
                       dim3(256), stream, reinterpret_cast<const uint16_t*>(h), P, (int)I,
                       reinterpret_cast<uint16_t*>(a));
}

hipError_t launch_moe_combine(const void* o, const float* w, int64_t T, int64_t topk, int64_t H, void* out,
                              hipStream_t stream) {
  const int64_t vecs = T * H / 8;
  return launch_kernel((const void*)moe_combine_kernel, dim3((unsigned)std::max<int64_t>(1, (vecs + 255) / 256)),
                       dim3(256), stream, reinterpret_cast<const uint16_t*>(o), w, T, (int)topk, (int)H,
                       reinterpret_cast<uint16_t*>(out));
}

}  // namespace nvfp4
