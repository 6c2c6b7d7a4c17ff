// NVFP4 W4A4 on gfx950: activations quantized to NVFP4 at run time with a
// static global input scale, then the product of the two NVFP4 operands.
//
// Method: vLLM modelopt.py, KNvfp4Dynamic (static global input scale, per-16
// block scales computed at run time), maybe_fuse_global_scales (alpha =
// input_global_scale * weight_global_scale) and the NVFP4 recipe (static FP4
// weight, dynamic FP4 activation); the block-scale and code rules are those of
// the weight quantizer (vLLM API docs, quantization.online.lm_head,
// _quantize_nvfp4).
//
// Design.  gfx950's block-scaled MFMA takes E2M1 operands with one E8M0
// (power-of-two) scale per 32 values; NVFP4 has an E4M3 scale per 16, whose
// mantissa the instruction cannot apply, so the product does not map onto it.
// Instead both operands are dequantized exactly: code * block scale has at
// most 6 significant bits and lies in [2^-10, 2688], so it is a bf16 value,
// and the W4A16 kernels already multiply bf16 activations by such weights
// with exact float32 products.  The activation is dequantized once into a
// caller-provided bf16 workspace (2 M K bytes, small next to the weight), the
// GEMM then runs unchanged with alpha in place of the weight's global scale.
//
// w4a4_dequant_x_kernel: one thread per 32-bit code word (8 codes, half a
//   block): 8 bf16 values code * scale, one 16-byte store; the first thread
//   also writes alpha = fl32(gs_in * gs_w) after the values.
#include <algorithm>
#include <mutex>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {

__global__ __launch_bounds__(256) void w4a4_dequant_x_kernel(const uint32_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales, int64_t nwords,
                                                             const float* __restrict__ gs_in,
                                                             const float* __restrict__ gs_w,
                                                             bf16x8* __restrict__ xd, float* __restrict__ alpha) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *alpha = *gs_in * *gs_w;
  if (i >= nwords) return;
  const float s = NVFP4_E4M3_TO_F32((uint32_t)scales[i >> 1], 0);
  xd[i] = dequant8(packed[i], s);
}

// Scratch of nvfp4_w4a4_gemm_noalloc: the workspace of nvfp4_w4a4_gemm
// (dequantized activations, then alpha) in static device memory, for callers
// that cannot allocate.  Each device holds its own copy until the process
// ends.  In host code `scratch` only names the symbol: its device address on
// the current device comes from hipGetSymbolAddress, looked up once per
// device and cached; kernels receive that address.
static __device__ __align__(256) uint8_t scratch[kW4a4ScratchBytes];

hipError_t w4a4_scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_w4a4_dequant_x(const uint8_t* x_packed, const uint8_t* x_scales, int64_t M, int64_t K,
                                 const float* gs_in, const float* gs_w, void* xd, float* alpha,
                                 hipStream_t stream) {
  const int64_t nwords = M * K / 8;
  const int64_t blocks = (nwords + 255) / 256;
  return launch_kernel((const void*)w4a4_dequant_x_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256),
                       stream, reinterpret_cast<const uint32_t*>(x_packed), x_scales, nwords, gs_in, gs_w,
                       reinterpret_cast<bf16x8*>(xd), alpha);
}

}  // namespace nvfp4
