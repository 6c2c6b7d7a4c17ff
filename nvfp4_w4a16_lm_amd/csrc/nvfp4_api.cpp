// C-ABI entry points: host-side validation, then stream-ordered launches.
// No HIP API call happens before an argument check has passed.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/nvfp4_w4a16.h"
#include "nvfp4_launch.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

constexpr int64_t kMaxDim = (int64_t)1 << 30;        // per-dimension bound (int32 kernel indexing)
constexpr int64_t kMaxElems = (int64_t)1 << 40;      // N*K bound (64-bit flat offsets)
constexpr int64_t kMaxPrefillM = (int64_t)65535 * 128;  // grid.y limit of the prefill kernel
constexpr int64_t kMaxPartitions = (int64_t)1 << 20;     // partition scales per checkpoint tensor

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nvfp4_status check_weight_shape(int64_t N, int64_t K) {
  if (N < 1 || K < NVFP4_GROUP || K % NVFP4_GROUP != 0) return NVFP4_ERR_SHAPE;
  if (N > kMaxDim || K > kMaxDim || N * K > kMaxElems) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

nvfp4_status validate_quantize(const void* W, int64_t N, int64_t K, const uint8_t* packed,
                               const uint8_t* scales, const float* gs) {
  if (!W || !packed || !scales || !gs) return NVFP4_ERR_NULL;
  const nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(gs, 4))
    return NVFP4_ERR_ALIGN;
  const Range rw = span(W, N * K * 2), rp = span(packed, N * K / 2), rs = span(scales, N * K / 16),
              rg = span(gs, 4);
  if (overlap(rw, rp) || overlap(rw, rs) || overlap(rw, rg) || overlap(rp, rs) || overlap(rp, rg) ||
      overlap(rs, rg))
    return NVFP4_ERR_ALIAS;
  return NVFP4_OK;
}

nvfp4_status finish(hipError_t e) {
  if (e == hipSuccess) return NVFP4_OK;
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return NVFP4_ERR_LAUNCH;
}

nvfp4_status run_quantize(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                          float* global_scale, void* stream) {
  const nvfp4_status s = validate_quantize(W, N, K, packed, scales, global_scale);
  if (s != NVFP4_OK) return s;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_quantize(W, N, K, packed, scales, global_scale, (hipStream_t)stream));
}

// nvfp4_w4a4_gemm with a caller workspace, or (use_scratch) with the
// library's static scratch; validation first, then the two launches.
nvfp4_status run_w4a4(const uint8_t* x_packed, const uint8_t* x_scales, const float* input_global_scale, int64_t M,
                      int64_t K, const uint8_t* packed, const uint8_t* scales, const float* global_scale, int64_t N,
                      const void* bias, void* workspace, bool use_scratch, void* y, void* stream) {
  if (!packed || !scales || !global_scale ||
      (M != 0 && (!x_packed || !x_scales || !input_global_scale || (!use_scratch && !workspace) || !y)))
    return NVFP4_ERR_NULL;
  nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (M < 0 || M > kMaxPrefillM || M * K > kMaxElems || M * N > kMaxElems) return NVFP4_ERR_SHAPE;
  const int64_t ws_bytes = 2 * M * K + 16;
  if (use_scratch && ws_bytes > nvfp4::kW4a4ScratchBytes) return NVFP4_ERR_SCRATCH;
  if (M == 0) return NVFP4_OK;
  if (!aligned(x_packed, 16) || !aligned(x_scales, 4) || !aligned(input_global_scale, 4) || !aligned(packed, 16) ||
      !aligned(scales, 4) || !aligned(global_scale, 4) || (!use_scratch && !aligned(workspace, 16)) ||
      !aligned(y, 16) || (bias && !aligned(bias, 2)))
    return NVFP4_ERR_ALIGN;
  const Range ry = span(y, M * N * 2);
  const Range ins[] = {span(x_packed, M * K / 2), span(x_scales, M * K / 16), span(input_global_scale, 4),
                       span(packed, N * K / 2),   span(scales, N * K / 16),   span(global_scale, 4),
                       span(bias ? bias : y, bias ? N * 2 : 0)};
  for (const Range& r : ins)
    if (overlap(ry, r)) return NVFP4_ERR_ALIAS;
  if (!use_scratch) {
    const Range rw = span(workspace, ws_bytes);
    if (overlap(ry, rw)) return NVFP4_ERR_ALIAS;
    for (const Range& r : ins)
      if (overlap(rw, r)) return NVFP4_ERR_ALIAS;
  }
  g_last_hip_error[0] = '\0';
  if (use_scratch) {
    const hipError_t e = nvfp4::w4a4_scratch_address(&workspace);
    if (e != hipSuccess) return finish(e);
  }
  const hipStream_t st = (hipStream_t)stream;
  uint8_t* const xd = static_cast<uint8_t*>(workspace);
  float* const alpha = reinterpret_cast<float*>(xd + 2 * M * K);
  hipError_t e = nvfp4::launch_w4a4_dequant_x(x_packed, x_scales, M, K, input_global_scale, global_scale, xd,
                                              alpha, st);
  if (e != hipSuccess) return finish(e);
  if (M <= nvfp4::kDecodeMaxM) return finish(nvfp4::launch_gemv(xd, M, K, packed, scales, alpha, N, bias, y, st));
  return finish(nvfp4::launch_gemm_prefill(xd, M, K, packed, scales, alpha, N, bias, y, st));
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                            float* global_scale, void* stream) {
  return run_quantize(W, N, K, packed, scales, global_scale, stream);
}

nvfp4_status nvfp4_refresh_inplace(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                                   float* global_scale, void* stream) {
  // The same kernels write the same bytes; the sequence holds no allocation
  // and no memset node, so graphs captured on these buffers stay valid.
  return run_quantize(W, N, K, packed, scales, global_scale, stream);
}

nvfp4_status nvfp4_w4a16_gemm(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                              const uint8_t* scales, const float* global_scale, int64_t N,
                              const void* bias, void* y, void* stream) {
  // x and y may be NULL when M == 0 (an empty activation tensor has no storage).
  if (!packed || !scales || !global_scale || (M != 0 && (!x || !y))) return NVFP4_ERR_NULL;
  nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (M < 0 || M > kMaxPrefillM || M * K > kMaxElems || M * N > kMaxElems) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(packed, 16) || !aligned(scales, 4) ||
      !aligned(global_scale, 4) || (bias && !aligned(bias, 2)))
    return NVFP4_ERR_ALIGN;
  const Range ry = span(y, M * N * 2);
  if (M > 0 && (overlap(ry, span(x, M * K * 2)) || overlap(ry, span(packed, N * K / 2)) ||
                overlap(ry, span(scales, N * K / 16)) || overlap(ry, span(global_scale, 4)) ||
                (bias && overlap(ry, span(bias, N * 2)))))
    return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  const hipStream_t st = (hipStream_t)stream;
  if (M <= nvfp4::kDecodeMaxM)
    return finish(nvfp4::launch_gemv(x, M, K, packed, scales, global_scale, N, bias, y, st));
  return finish(nvfp4::launch_gemm_prefill(x, M, K, packed, scales, global_scale, N, bias, y, st));
}

nvfp4_status nvfp4_import_checkpoint(const float* partition_scales, int64_t num_partitions, int convention,
                                     const uint8_t* scales, int64_t N, int64_t K, float* global_scale,
                                     uint32_t* flags, void* stream) {
  if (!partition_scales || !scales || !global_scale || !flags) return NVFP4_ERR_NULL;
  if (convention != NVFP4_SCALE2_MODELOPT && convention != NVFP4_SCALE2_COMPRESSED_TENSORS) return NVFP4_ERR_ARG;
  nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (num_partitions < 1 || num_partitions > kMaxPartitions) return NVFP4_ERR_SHAPE;
  if (!aligned(partition_scales, 4) || !aligned(scales, 16) || !aligned(global_scale, 4) || !aligned(flags, 4))
    return NVFP4_ERR_ALIGN;
  const Range rp = span(partition_scales, num_partitions * 4), rs = span(scales, N * K / 16),
              rg = span(global_scale, 4), rf = span(flags, 4);
  if (overlap(rg, rp) || overlap(rg, rs) || overlap(rf, rp) || overlap(rf, rs) || overlap(rg, rf))
    return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_import(partition_scales, num_partitions, convention, scales, N * K / 16,
                                     global_scale, flags, (hipStream_t)stream));
}

nvfp4_status nvfp4_fill_scale_sentinel(uint8_t* scales, int64_t N, int64_t K, void* stream) {
  if (!scales) return NVFP4_ERR_NULL;
  const nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (!aligned(scales, 16)) return NVFP4_ERR_ALIGN;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_fill_sentinel(scales, N * K / 16, (hipStream_t)stream));
}

nvfp4_status nvfp4_fp8_quantize_rows(const void* A, int64_t R, int64_t K, uint8_t* q, float* row_scales,
                                     void* stream) {
  if (!A || !q || !row_scales) return NVFP4_ERR_NULL;
  const nvfp4_status s = check_weight_shape(R, K);
  if (s != NVFP4_OK) return s;
  if (!aligned(A, 16) || !aligned(q, 16) || !aligned(row_scales, 4)) return NVFP4_ERR_ALIGN;
  const Range ra = span(A, R * K * 2), rq = span(q, R * K), rs = span(row_scales, R * 4);
  if (overlap(ra, rq) || overlap(ra, rs) || overlap(rq, rs)) return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_fp8_quant_rows(A, R, K, q, row_scales, (hipStream_t)stream));
}

nvfp4_status nvfp4_fp8_gemm(const uint8_t* xq, const float* x_scales, int64_t M, int64_t K, const uint8_t* wq,
                            const float* w_scales, int64_t N, const void* bias, void* y, void* stream) {
  if (!wq || !w_scales || (M != 0 && (!xq || !x_scales || !y))) return NVFP4_ERR_NULL;
  const nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (M < 0 || M > kMaxPrefillM || M * K > kMaxElems || M * N > kMaxElems) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(x_scales, 4) ||
      !aligned(w_scales, 4) || (bias && !aligned(bias, 2)))
    return NVFP4_ERR_ALIGN;
  const Range ry = span(y, M * N * 2);
  if (overlap(ry, span(xq, M * K)) || overlap(ry, span(x_scales, M * 4)) || overlap(ry, span(wq, N * K)) ||
      overlap(ry, span(w_scales, N * 4)) || (bias && overlap(ry, span(bias, N * 2))))
    return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_fp8_gemm(xq, x_scales, M, K, wq, w_scales, N, bias, y, (hipStream_t)stream));
}

nvfp4_status nvfp4_quantize_activations(const void* x, int64_t M, int64_t K, const float* input_global_scale,
                                        uint8_t* packed, uint8_t* scales, void* stream) {
  if (!x || !input_global_scale || !packed || !scales) return NVFP4_ERR_NULL;
  const nvfp4_status s = check_weight_shape(M, K);
  if (s != NVFP4_OK) return s;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(input_global_scale, 4))
    return NVFP4_ERR_ALIGN;
  const Range rx = span(x, M * K * 2), rg = span(input_global_scale, 4), rp = span(packed, M * K / 2),
              rs = span(scales, M * K / 16);
  if (overlap(rp, rx) || overlap(rp, rg) || overlap(rs, rx) || overlap(rs, rg) || overlap(rp, rs))
    return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_quantize_given_scale(x, M, K, input_global_scale, packed, scales,
                                                   (hipStream_t)stream));
}

int64_t nvfp4_w4a4_workspace_bytes(int64_t M, int64_t K) { return (M < 0 || K < 0) ? 0 : 2 * M * K + 16; }

nvfp4_status nvfp4_w4a4_gemm(const uint8_t* x_packed, const uint8_t* x_scales, const float* input_global_scale,
                             int64_t M, int64_t K, const uint8_t* packed, const uint8_t* scales,
                             const float* global_scale, int64_t N, const void* bias, void* workspace, void* y,
                             void* stream) {
  return run_w4a4(x_packed, x_scales, input_global_scale, M, K, packed, scales, global_scale, N, bias, workspace,
                  false, y, stream);
}

nvfp4_status nvfp4_w4a4_gemm_noalloc(const uint8_t* x_packed, const uint8_t* x_scales,
                                     const float* input_global_scale, int64_t M, int64_t K, const uint8_t* packed,
                                     const uint8_t* scales, const float* global_scale, int64_t N, const void* bias,
                                     void* y, void* stream) {
  return run_w4a4(x_packed, x_scales, input_global_scale, M, K, packed, scales, global_scale, N, bias, nullptr,
                  true, y, stream);
}

// ---------------------------------------------------------------------------
// Mixture of experts (W4A16)
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

constexpr int64_t kMaxExperts = 65534;               // grid.y of the grouped GEMM is E + 1
constexpr int64_t kMaxPairs = (int64_t)1 << 28;

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

nvfp4_status check_experts(int64_t E, int64_t N, int64_t K) {
  if (E < 1 || E > kMaxExperts) return NVFP4_ERR_SHAPE;
  const nvfp4_status s = check_weight_shape(N, K);
  if (s != NVFP4_OK) return s;
  if (E * N > kMaxDim || E * N * K > kMaxElems) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int64_t nvfp4_moe_gemm_workspace_bytes(int64_t P, int64_t E) {
  return (P < 0 || E < 1) ? 0 : nvfp4::moe_route_bytes(P, E);
}

int64_t nvfp4_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I) {
  if (T < 0 || topk < 1 || E < 1 || H < 0 || I < 0) return 0;
  const int64_t P = T * topk;
  return round256(nvfp4::moe_route_bytes(P, E)) + round256(P * 2 * I * 2) + round256(P * I * 2) +
         round256(P * H * 2);
}

nvfp4_status nvfp4_moe_w4a16_gemm(const void* x, int64_t x_rows, int64_t K, const int32_t* topk_ids, int64_t P,
                                  int64_t row_div, const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scales, int64_t E, int64_t N, void* workspace, void* y,
                                  uint32_t* invalid_pairs, void* stream) {
  if (!packed || !scales || !global_scales || (P != 0 && (!x || !topk_ids || !workspace || !y)))
    return NVFP4_ERR_NULL;
  nvfp4_status s = check_experts(E, N, K);
  if (s != NVFP4_OK) return s;
  if (P < 0 || P > kMaxPairs || row_div < 1 || x_rows < 0 || x_rows > kMaxDim || x_rows * K > kMaxElems ||
      P * N > kMaxElems || (P + row_div - 1) / row_div > x_rows)
    return NVFP4_ERR_SHAPE;
  if (P == 0) return NVFP4_OK;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(packed, 16) || !aligned(global_scales, 4) ||
      !aligned(topk_ids, 4) || !aligned(workspace, 16) || (invalid_pairs && !aligned(invalid_pairs, 4)))
    return NVFP4_ERR_ALIGN;
  const Range ry = span(y, P * N * 2), rw = span(workspace, nvfp4_moe_gemm_workspace_bytes(P, E)),
              ri = span(invalid_pairs, invalid_pairs ? 4 : 0);
  const Range ins[] = {span(x, x_rows * K * 2), span(topk_ids, P * 4), span(packed, E * N * K / 2),
                       span(scales, E * N * K / 16), span(global_scales, E * 4)};
  if (overlap(ry, rw) || overlap(ry, ri) || overlap(rw, ri)) return NVFP4_ERR_ALIAS;
  for (const Range& r : ins)
    if (overlap(ry, r) || overlap(rw, r) || overlap(ri, r)) return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  const hipStream_t st = (hipStream_t)stream;
  int32_t* const route = static_cast<int32_t*>(workspace);
  hipError_t e = nvfp4::launch_moe_route(topk_ids, P, E, route, invalid_pairs, st);
  if (e != hipSuccess) return finish(e);
  return finish(nvfp4::launch_moe_gemm(x, row_div, K, route, P, packed, scales, global_scales, E, N, y, st));
}

nvfp4_status nvfp4_moe_silu_and_mul(const void* h, int64_t P, int64_t I, void* a, void* stream) {
  if (P != 0 && (!h || !a)) return NVFP4_ERR_NULL;
  if (P < 0 || P > kMaxPairs || I < 8 || I % 8 != 0 || I > kMaxDim || P * 2 * I > kMaxElems)
    return NVFP4_ERR_SHAPE;
  if (P == 0) return NVFP4_OK;
  if (!aligned(h, 16) || !aligned(a, 16)) return NVFP4_ERR_ALIGN;
  if (overlap(span(h, P * 2 * I * 2), span(a, P * I * 2))) return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_moe_silu_mul(h, P, I, a, (hipStream_t)stream));
}

nvfp4_status nvfp4_moe_combine(const void* o, const float* topk_weights, int64_t T, int64_t topk, int64_t H,
                               void* out, void* stream) {
  if (T != 0 && (!o || !topk_weights || !out)) return NVFP4_ERR_NULL;
  if (T < 0 || topk < 1 || T * topk > kMaxPairs || H < 8 || H % 8 != 0 || H > kMaxDim ||
      T * topk * H > kMaxElems)
    return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!aligned(o, 16) || !aligned(out, 16) || !aligned(topk_weights, 4)) return NVFP4_ERR_ALIGN;
  const Range rout = span(out, T * H * 2);
  if (overlap(rout, span(o, T * topk * H * 2)) || overlap(rout, span(topk_weights, T * topk * 4)))
    return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  return finish(nvfp4::launch_moe_combine(o, topk_weights, T, topk, H, out, (hipStream_t)stream));
}

nvfp4_status nvfp4_moe_w4a16_forward(const void* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                     const float* topk_weights, int64_t topk, const uint8_t* w13_packed,
                                     const uint8_t* w13_scales, const float* w13_global_scales,
                                     const uint8_t* w2_packed, const uint8_t* w2_scales,
                                     const float* w2_global_scales, int64_t E, int64_t I, void* workspace,
                                     void* out, uint32_t* invalid_pairs, void* stream) {
  if (!w13_packed || !w13_scales || !w13_global_scales || !w2_packed || !w2_scales || !w2_global_scales ||
      (T != 0 && (!x || !topk_ids || !topk_weights || !workspace || !out)))
    return NVFP4_ERR_NULL;
  if (T < 0 || topk < 1 || T > kMaxDim || T * topk > kMaxPairs) return NVFP4_ERR_SHAPE;
  nvfp4_status s = check_experts(E, 2 * I, H);
  if (s != NVFP4_OK) return s;
  s = check_experts(E, H, I);
  if (s != NVFP4_OK) return s;
  const int64_t P = T * topk;
  if (P * 2 * I > kMaxElems || P * H > kMaxElems) return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w13_packed, 16) || !aligned(w2_packed, 16) ||
      !aligned(w13_global_scales, 4) || !aligned(w2_global_scales, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_weights, 4) || !aligned(workspace, 16) || (invalid_pairs && !aligned(invalid_pairs, 4)))
    return NVFP4_ERR_ALIGN;
  const int64_t ws_bytes = nvfp4_moe_workspace_bytes(T, topk, E, H, I);
  const Range rout = span(out, T * H * 2), rw = span(workspace, ws_bytes),
              ri = span(invalid_pairs, invalid_pairs ? 4 : 0);
  const Range ins[] = {span(x, T * H * 2),
                       span(topk_ids, P * 4),
                       span(topk_weights, P * 4),
                       span(w13_packed, E * 2 * I * H / 2),
                       span(w13_scales, E * 2 * I * H / 16),
                       span(w13_global_scales, E * 4),
                       span(w2_packed, E * H * I / 2),
                       span(w2_scales, E * H * I / 16),
                       span(w2_global_scales, E * 4)};
  if (overlap(rout, rw) || overlap(rout, ri) || overlap(rw, ri)) return NVFP4_ERR_ALIAS;
  for (const Range& r : ins)
    if (overlap(rout, r) || overlap(rw, r) || overlap(ri, r)) return NVFP4_ERR_ALIAS;
  g_last_hip_error[0] = '\0';
  const hipStream_t st = (hipStream_t)stream;
  uint8_t* const base = static_cast<uint8_t*>(workspace);
  int32_t* const route = reinterpret_cast<int32_t*>(base);
  uint8_t* const h = base + round256(nvfp4::moe_route_bytes(P, E));
  uint8_t* const a = h + round256(P * 2 * I * 2);
  uint8_t* const o = a + round256(P * I * 2);
  hipError_t e = nvfp4::launch_moe_route(topk_ids, P, E, route, invalid_pairs, st);
  if (e == hipSuccess)
    e = nvfp4::launch_moe_gemm(x, topk, H, route, P, w13_packed, w13_scales, w13_global_scales, E, 2 * I, h, st);
  if (e == hipSuccess) e = nvfp4::launch_moe_silu_mul(h, P, I, a, st);
  if (e == hipSuccess)
    e = nvfp4::launch_moe_gemm(a, 1, I, route, P, w2_packed, w2_scales, w2_global_scales, E, H, o, st);
  if (e == hipSuccess) e = nvfp4::launch_moe_combine(o, topk_weights, T, topk, H, out, st);
  return finish(e);
}

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (need N >= 1, K >= 16, K % 16 == 0, M >= 0, sizes in range)";
    case NVFP4_ERR_ALIGN:
      return "misaligned pointer (W, x, y, packed: 16 B; scales: 4 B, 16 B for the import calls; "
             "global_scale, flags, partition scales: 4 B; bias: 2 B)";
    case NVFP4_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case NVFP4_ERR_LAUNCH: return "HIP error while enqueueing (see nvfp4_last_hip_error)";
    case NVFP4_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
    case NVFP4_ERR_ARG: return "an enumerated argument is out of range";
    default: return "unknown status";
  }
}

const char* nvfp4_last_hip_error(void) { return g_last_hip_error; }

int nvfp4_abi_version(void) { return 4; }

}  // extern "C"
