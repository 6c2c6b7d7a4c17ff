// Internal launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

namespace nvfp4 {

// hipLaunchKernel with a typed argument pack.  The argument types must match
// the kernel's parameter types exactly (callers cast at the call site).
// Returns the launch's own status.
template <typename... Args>
inline hipError_t launch_kernel_lds(const void* fn, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                    Args... args) {
  void* argv[] = {(void*)&args..., nullptr};
  return hipLaunchKernel(fn, grid, block, argv, lds, stream);
}

template <typename... Args>
inline hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  return launch_kernel_lds(fn, grid, block, 0, stream, args...);
}

// The current device (0 if the query fails).
inline int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

// Compute units of device dev, queried once per device (256 if the query fails;
// a failed query is not cached and its error is cleared so that it cannot be
// reported by a later launch check).
inline int device_cus(int dev) {
  static std::atomic<int> cache[64];
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Resident workgroups per compute unit of kernel fn with `block` threads and
// `lds` bytes of dynamic LDS on device dev, queried once per (kernel, device,
// block, lds) (1 if the query fails; not cached, error cleared).
inline int blocks_per_cu(const void* fn, int dev, int block, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int, size_t>, int> cache;
  const auto key = std::make_tuple(fn, dev, block, lds);
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, lds) != hipSuccess || per_cu <= 0) {
    (void)hipGetLastError();
    return 1;
  }
  std::lock_guard<std::mutex> g(mu);
  cache[key] = per_cu;
  return per_cu;
}

// Raise kernel fn's dynamic LDS limit to `bytes` once per (kernel, device)
// (the default allows less than the hardware's 160 KiB).  Concurrent first
// calls may both set it, which is harmless.
inline hipError_t ensure_dynamic_lds(const void* fn, int dev, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> done;
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = done.find({fn, dev});
    if (it != done.end() && it->second >= bytes) return hipSuccess;
  }
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  int& v = done[{fn, dev}];
  if (v < bytes) v = bytes;
  return hipSuccess;
}

// Quantization: amax -> global scale -> block scales + packed codes.
hipError_t launch_quantize(const void* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* scales,
                           float* global_scale, hipStream_t stream);

// y[M,N] = x[M,K] . dequant(W)^T (+ bias); M <= 64 streaming decode kernel.
hipError_t launch_gemv(const void* x, int64_t M, int64_t K, const uint8_t* packed, const uint8_t* scales,
                       const float* global_scale, int64_t N, const void* bias, void* y, hipStream_t stream);

// Same for M > 64: LDS-staged dequant + bf16 MFMA.
hipError_t launch_gemm_prefill(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                               const uint8_t* scales, const float* global_scale, int64_t N,
                               const void* bias, void* y, hipStream_t stream);

constexpr int64_t kDecodeMaxM = 64;

// Checkpoint import: collapse the partition scales into the global scale and
// write the flags word, then scan the nbytes block-scale bytes for NaN.
hipError_t launch_import(const float* partition_scales, int64_t P, int convention, const uint8_t* scales,
                         int64_t nbytes, float* global_scale, uint32_t* flags, hipStream_t stream);

// Fill nbytes block-scale bytes with the e4m3fn NaN sentinel 0x7F.
hipError_t launch_fill_sentinel(uint8_t* scales, int64_t nbytes, hipStream_t stream);

// FP8 copy: row-wise E4M3 quantization of a bf16 [R, K] matrix, and the
// scaled FP8 GEMM y = bf16(s_x[m] s_w[n] sum_k xq wq (+ bias)).
hipError_t launch_fp8_quant_rows(const void* a, int64_t R, int64_t K, uint8_t* q, float* scales,
                                 hipStream_t stream);
// W4A4: NVFP4 quantization of activations with a given global scale, and the
// exact bf16 dequantization of them (code * block scale) plus alpha.
hipError_t launch_quantize_given_scale(const void* X, int64_t M, int64_t K, const float* global_scale,
                                       uint8_t* packed, uint8_t* scales, hipStream_t stream);
hipError_t launch_w4a4_dequant_x(const uint8_t* x_packed, const uint8_t* x_scales, int64_t M, int64_t K,
                                 const float* gs_in, const float* gs_w, void* xd, float* alpha,
                                 hipStream_t stream);
// Static scratch of the no-allocation W4A4 call: its size (the largest
// workspace it serves, 2 M K + 16 bytes) and its device address on the
// current device (looked up once per device).
constexpr int64_t kW4a4ScratchBytes = (int64_t)4 << 20;
constexpr int kMaxDevices = 64;
hipError_t w4a4_scratch_address(void** out);
hipError_t launch_fp8_gemm(const uint8_t* xq, const float* xs, int64_t M, int64_t K, const uint8_t* wq,
                           const float* ws, int64_t N, const void* bias, void* y, hipStream_t stream);

// Mixture of experts (W4A16).  Routing workspace: int32 offsets of E + 1
// groups (the last one holds pairs with an id outside [0, E)) padded to a
// multiple of 4 words, then the P pair indices grouped by expert.
inline int64_t moe_route_offsets_words(int64_t E) { return (E + 2 + 3) / 4 * 4; }
inline int64_t moe_route_bytes(int64_t P, int64_t E) { return 4 * (moe_route_offsets_words(E) + (P + 3) / 4 * 4); }
hipError_t launch_moe_route(const int32_t* ids, int64_t P, int64_t E, int32_t* route_ws, uint32_t* invalid,
                            hipStream_t stream);
hipError_t launch_moe_gemm(const void* x, int64_t row_div, int64_t K, const int32_t* route_ws, int64_t P,
                           const uint8_t* packed, const uint8_t* scales, const float* gs, int64_t E, int64_t N,
                           void* y, hipStream_t stream);
// The x-resident decode kernel over the experts with 1..mcap pairs, on the
// routing table's offsets and order: its plan (mcap = 0: not used), then the
// launch.
struct MoeXresPlan {
  int mcap;   // largest pair count it takes
  int nw;     // wavefronts per workgroup
  int ks;     // wavefronts sharing one tile's K
  int depth;  // chunk regions per wavefront (0: one, refilled after the read; 2: the two-region pipeline)
};
MoeXresPlan moe_xres_plan(int64_t P, int64_t E, int64_t K, int64_t N);
hipError_t launch_moe_xres(const void* x, int64_t row_div, int64_t K, const int32_t* offsets, const int32_t* order,
                           const MoeXresPlan& plan, int64_t P, const uint8_t* packed, const uint8_t* scales,
                           const float* gs, int64_t E, int64_t N, void* y, hipStream_t stream);
// The panel decode kernel over the experts with mmin..mcap pairs, `rows`
// (16, 32 or 64) activation rows per pass over an expert's weights (at 16 or
// 32, experts with more pairs take several passes; at 64, mcap is at most
// 64); K % 512 == 0, otherwise nothing is launched.  With zero_rows it also writes the zero rows of the pairs whose
// id is outside [0, E).
hipError_t launch_moe_panel(const void* x, int64_t row_div, int64_t K, const int32_t* offsets, const int32_t* order,
                            int mmin, int mcap, int rows, int64_t P, const uint8_t* packed, const uint8_t* scales,
                            const float* gs, int64_t E, int64_t N, void* y, bool zero_rows, hipStream_t stream);
hipError_t launch_moe_silu_mul(const void* h, int64_t P, int64_t I, void* a, hipStream_t stream);
hipError_t launch_moe_combine(const void* o, const float* w, int64_t T, int64_t topk, int64_t H, void* out,
                              hipStream_t stream);

}  // namespace nvfp4
