"""ctypes binding of ``libnvfp4_w4a16.so`` (argument marshalling only).

Each function keeps the name of the C entry point it wraps.  torch is used for
device memory (allocating outputs, taking data pointers) and for the current
HIP stream; every step of the computation runs in the library's kernels.
There is no fallback: a missing library raises at first use.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_NAME = "libnvfp4_w4a16.so"
ABI_VERSION = 4

STATUS_NAMES = {
    0: "NVFP4_OK",
    1: "NVFP4_ERR_NULL",
    2: "NVFP4_ERR_SHAPE",
    3: "NVFP4_ERR_ALIGN",
    4: "NVFP4_ERR_ALIAS",
    5: "NVFP4_ERR_LAUNCH",
    6: "NVFP4_ERR_ARG",
    7: "NVFP4_ERR_SCRATCH",
}

#: Scale conventions of nvfp4_import_checkpoint (nvfp4_scale2_convention).
SCALE2_CONVENTIONS = {"modelopt": 0, "compressed-tensors": 1}

#: Flag bits written by nvfp4_import_checkpoint.
IMPORT_SCALES_NOT_LOADED = 1
IMPORT_PARTITIONS_DIFFER = 2
IMPORT_BAD_GLOBAL_SCALE = 4

#: Entry points declared in include/nvfp4_w4a16.h.
EXPORTED = ("nvfp4_quantize", "nvfp4_refresh_inplace", "nvfp4_w4a16_gemm",
            "nvfp4_fill_scale_sentinel", "nvfp4_import_checkpoint",
            "nvfp4_fp8_quantize_rows", "nvfp4_fp8_gemm",
            "nvfp4_quantize_activations", "nvfp4_w4a4_workspace_bytes", "nvfp4_w4a4_gemm",
            "nvfp4_w4a4_gemm_noalloc",
            "nvfp4_moe_gemm_workspace_bytes", "nvfp4_moe_w4a16_gemm", "nvfp4_moe_silu_and_mul",
            "nvfp4_moe_combine", "nvfp4_moe_workspace_bytes", "nvfp4_moe_w4a16_forward",
            "nvfp4_status_string", "nvfp4_last_hip_error", "nvfp4_abi_version")


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{fn}: {name}{': ' + detail if detail else ''}")


class NVFP4ShapeError(NVFP4Error, ValueError):
    """Bad shape (e.g. K not a multiple of 16), raised as a ValueError too."""


_lib = None


def library_path() -> str:
    return os.environ.get("NVFP4_W4A16_LIB",
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME))


def load_library() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m nvfp4_w4a16_lm_amd.build_lib` "
                          "(the NVFP4 path has no fallback)")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("nvfp4_quantize", "nvfp4_refresh_inplace"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        fn.restype = ctypes.c_int
    lib.nvfp4_w4a16_gemm.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, vp, vp]
    lib.nvfp4_w4a16_gemm.restype = ctypes.c_int
    lib.nvfp4_fill_scale_sentinel.argtypes = [vp, i64, i64, vp]
    lib.nvfp4_fill_scale_sentinel.restype = ctypes.c_int
    lib.nvfp4_import_checkpoint.argtypes = [vp, i64, ctypes.c_int, vp, i64, i64, vp, vp, vp]
    lib.nvfp4_import_checkpoint.restype = ctypes.c_int
    lib.nvfp4_fp8_quantize_rows.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.nvfp4_fp8_quantize_rows.restype = ctypes.c_int
    lib.nvfp4_fp8_gemm.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
    lib.nvfp4_fp8_gemm.restype = ctypes.c_int
    lib.nvfp4_quantize_activations.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.nvfp4_quantize_activations.restype = ctypes.c_int
    lib.nvfp4_w4a4_workspace_bytes.argtypes = [i64, i64]
    lib.nvfp4_w4a4_workspace_bytes.restype = i64
    lib.nvfp4_w4a4_gemm.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.nvfp4_w4a4_gemm.restype = ctypes.c_int
    lib.nvfp4_w4a4_gemm_noalloc.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i64, vp, vp, vp]
    lib.nvfp4_w4a4_gemm_noalloc.restype = ctypes.c_int
    lib.nvfp4_moe_gemm_workspace_bytes.argtypes = [i64, i64]
    lib.nvfp4_moe_gemm_workspace_bytes.restype = i64
    lib.nvfp4_moe_w4a16_gemm.argtypes = [vp, i64, i64, vp, i64, i64, vp, vp, vp, i64, i64, vp, vp, vp, vp]
    lib.nvfp4_moe_w4a16_gemm.restype = ctypes.c_int
    lib.nvfp4_moe_silu_and_mul.argtypes = [vp, i64, i64, vp, vp]
    lib.nvfp4_moe_silu_and_mul.restype = ctypes.c_int
    lib.nvfp4_moe_combine.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.nvfp4_moe_combine.restype = ctypes.c_int
    lib.nvfp4_moe_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.nvfp4_moe_workspace_bytes.restype = i64
    lib.nvfp4_moe_w4a16_forward.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp,
                                            vp, vp]
    lib.nvfp4_moe_w4a16_forward.restype = ctypes.c_int
    lib.nvfp4_status_string.argtypes = [ctypes.c_int]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_last_hip_error.argtypes = []
    lib.nvfp4_last_hip_error.restype = ctypes.c_char_p
    lib.nvfp4_abi_version.argtypes = []
    lib.nvfp4_abi_version.restype = ctypes.c_int
    if lib.nvfp4_abi_version() != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {lib.nvfp4_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status == 0:
        return
    lib = load_library()
    detail = lib.nvfp4_status_string(status).decode()
    if status == 5:
        detail += " -- " + lib.nvfp4_last_hip_error().decode()
    if status == 2:
        raise NVFP4ShapeError(fn, status, detail)
    raise NVFP4Error(fn, status, detail)


def _stream_of(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _as_bf16_2d(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{what} must be bfloat16, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    return t.contiguous()


def _check_out(t: torch.Tensor, shape, dtypes, device, what: str) -> None:
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or t.device != device or not t.is_contiguous():
        raise ValueError(f"{what}: expected contiguous {shape} {dtypes[0]} on {device}, "
                         f"got {tuple(t.shape)} {t.dtype} on {t.device}")


def nvfp4_quantize(weight: torch.Tensor, stream=None):
    """bf16 [N, K] -> (packed uint8 [N, K/2], scales float8_e4m3fn [N, K/16], global_scale fp32 [])."""
    w = _as_bf16_2d(weight, "weight")
    n, k = w.shape
    dev = w.device
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, k // 16), dtype=torch.float8_e4m3fn, device=dev)
    gs = torch.empty((), dtype=torch.float32, device=dev)
    lib = load_library()
    _check("nvfp4_quantize", lib.nvfp4_quantize(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(gs),
                                                _stream_of(w, stream)))
    return packed, scales, gs


def nvfp4_refresh_inplace(weight: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                          global_scale: torch.Tensor, stream=None) -> None:
    """Re-quantize ``weight`` into the existing buffers (pointers unchanged)."""
    w = _as_bf16_2d(weight, "weight")
    n, k = w.shape
    dev = w.device
    _check_out(packed, (n, k // 2), (torch.uint8,), dev, "packed")
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "scales")
    if global_scale.numel() != 1 or global_scale.dtype != torch.float32 or global_scale.device != dev:
        raise ValueError("global_scale must be one float32 on the weight's device")
    lib = load_library()
    _check("nvfp4_refresh_inplace",
           lib.nvfp4_refresh_inplace(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(global_scale),
                                     _stream_of(w, stream)))


def nvfp4_w4a16_gemm(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                     global_scale: torch.Tensor, bias: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 x [M, K] . dequant(W)^T (+ bias) -> bf16 [M, N]."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    if packed.dim() != 2 or packed.shape[1] * 2 != k:
        raise ValueError(f"packed shape {tuple(packed.shape)} does not match K={k}")
    n = packed.shape[0]
    dev = x.device
    _check_out(packed, (n, k // 2), (torch.uint8,), dev, "packed")
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "scales")
    if global_scale.numel() != 1 or global_scale.dtype != torch.float32 or global_scale.device != dev:
        raise ValueError("global_scale must be one float32 on x's device")
    if bias is not None:
        _check_out(bias, (n,), (torch.bfloat16,), dev, "bias")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, (m, n), (torch.bfloat16,), dev, "out")
    lib = load_library()
    _check("nvfp4_w4a16_gemm",
           lib.nvfp4_w4a16_gemm(_ptr(x), m, k, _ptr(packed), _ptr(scales), _ptr(global_scale), n,
                                _ptr(bias), _ptr(out), _stream_of(x, stream)))
    return out


class NVFP4NotLoadedError(RuntimeError):
    """Block scales still hold the NaN sentinel: the checkpoint never wrote them."""


def nvfp4_fill_scale_sentinel(scales: torch.Tensor, k: int, stream=None) -> None:
    """Fill a [N, K/16] block-scale buffer with the e4m3fn NaN sentinel 0x7F."""
    if scales.dim() != 2 or scales.shape[1] * 16 != k:
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match K={k}")
    n = scales.shape[0]
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), scales.device, "scales")
    lib = load_library()
    _check("nvfp4_fill_scale_sentinel",
           lib.nvfp4_fill_scale_sentinel(_ptr(scales), n, k, _stream_of(scales, stream)))


def nvfp4_import_checkpoint(partition_scales: torch.Tensor, scales: torch.Tensor, k: int,
                            convention: str, global_scale: torch.Tensor | None = None,
                            flags: torch.Tensor | None = None, stream=None):
    """Global scale (fp32 []) and flags (int32 [], NVFP4_IMPORT_* bits) of a
    pre-quantized checkpoint; both are device tensors, valid in stream order."""
    if convention not in SCALE2_CONVENTIONS:
        raise ValueError(f"convention must be one of {sorted(SCALE2_CONVENTIONS)}, got {convention!r}")
    if scales.dim() != 2 or scales.shape[1] * 16 != k:
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match K={k}")
    n = scales.shape[0]
    dev = scales.device
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "scales")
    ps = partition_scales.reshape(-1)
    if ps.dtype != torch.float32 or ps.device != dev or not ps.is_contiguous():
        raise ValueError("partition_scales must be contiguous float32 on the scales' device")
    if global_scale is None:
        global_scale = torch.empty((), dtype=torch.float32, device=dev)
    if flags is None:
        flags = torch.empty((), dtype=torch.int32, device=dev)
    if global_scale.numel() != 1 or global_scale.dtype != torch.float32 or global_scale.device != dev:
        raise ValueError("global_scale must be one float32 on the scales' device")
    if flags.numel() != 1 or flags.dtype != torch.int32 or flags.device != dev:
        raise ValueError("flags must be one int32 on the scales' device")
    lib = load_library()
    _check("nvfp4_import_checkpoint",
           lib.nvfp4_import_checkpoint(_ptr(ps), ps.numel(), SCALE2_CONVENTIONS[convention], _ptr(scales),
                                       n, k, _ptr(global_scale), _ptr(flags), _stream_of(scales, stream)))
    return global_scale, flags


def check_import_flags(flags: torch.Tensor, what: str = "lm_head") -> int:
    """Host-side reaction to the flags, as the checkpoint loaders react
    (synchronises): raise when block scales were never loaded or the global
    scale is unusable; warn when partitions had different global scales."""
    f = int(flags.item())
    if f & IMPORT_SCALES_NOT_LOADED:
        raise NVFP4NotLoadedError(f"NVFP4 block scales of {what} were never loaded (still NaN)")
    if f & IMPORT_BAD_GLOBAL_SCALE:
        raise NVFP4NotLoadedError(f"NVFP4 global scale of {what} is not a finite positive number")
    if f & IMPORT_PARTITIONS_DIFFER:
        import warnings
        warnings.warn(f"NVFP4 global scales differ across the fused partitions of {what}; "
                      "one (the largest) serves all of them, which may reduce accuracy")
    return f


def nvfp4_fp8_quantize_rows(a: torch.Tensor, q: torch.Tensor | None = None,
                            scales: torch.Tensor | None = None, stream=None):
    """bf16 [R, K] -> (float8_e4m3fn [R, K], float32 [R]): one E4M3 scale per
    row (per output row of a weight, per token of an activation)."""
    a = _as_bf16_2d(a, "a")
    r, k = a.shape
    dev = a.device
    if q is None:
        q = torch.empty((r, k), dtype=torch.float8_e4m3fn, device=dev)
    else:
        _check_out(q, (r, k), (torch.float8_e4m3fn, torch.uint8), dev, "q")
    if scales is None:
        scales = torch.empty((r,), dtype=torch.float32, device=dev)
    else:
        _check_out(scales, (r,), (torch.float32,), dev, "scales")
    lib = load_library()
    _check("nvfp4_fp8_quantize_rows",
           lib.nvfp4_fp8_quantize_rows(_ptr(a), r, k, _ptr(q), _ptr(scales), _stream_of(a, stream)))
    return q, scales


def nvfp4_fp8_gemm(xq: torch.Tensor, x_scales: torch.Tensor, wq: torch.Tensor, w_scales: torch.Tensor,
                   bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """bf16 [M, N] = x_scales[m] * w_scales[n] * (xq . wq^T) (+ bias)."""
    if xq.dim() != 2 or wq.dim() != 2 or xq.shape[1] != wq.shape[1]:
        raise ValueError(f"xq {tuple(xq.shape)} and wq {tuple(wq.shape)} must be [M, K] and [N, K]")
    m, k = xq.shape
    n = wq.shape[0]
    dev = wq.device
    _check_out(xq, (m, k), (torch.float8_e4m3fn, torch.uint8), dev, "xq")
    _check_out(wq, (n, k), (torch.float8_e4m3fn, torch.uint8), dev, "wq")
    _check_out(x_scales, (m,), (torch.float32,), dev, "x_scales")
    _check_out(w_scales, (n,), (torch.float32,), dev, "w_scales")
    if bias is not None:
        _check_out(bias, (n,), (torch.bfloat16,), dev, "bias")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, (m, n), (torch.bfloat16,), dev, "out")
    lib = load_library()
    _check("nvfp4_fp8_gemm",
           lib.nvfp4_fp8_gemm(_ptr(xq), _ptr(x_scales), m, k, _ptr(wq), _ptr(w_scales), n, _ptr(bias),
                              _ptr(out), _stream_of(wq, stream)))
    return out


def nvfp4_quantize_activations(x: torch.Tensor, input_global_scale: torch.Tensor, stream=None):
    """bf16 [M, K] -> (packed uint8 [M, K/2], scales float8_e4m3fn [M, K/16]) with a
    given global scale (fp32 [] on the device, dequantization direction)."""
    x = _as_bf16_2d(x, "x")
    m, k = x.shape
    dev = x.device
    if input_global_scale.numel() != 1 or input_global_scale.dtype != torch.float32 or \
            input_global_scale.device != dev:
        raise ValueError("input_global_scale must be one float32 on x's device")
    packed = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((m, k // 16), dtype=torch.float8_e4m3fn, device=dev)
    lib = load_library()
    _check("nvfp4_quantize_activations",
           lib.nvfp4_quantize_activations(_ptr(x), m, k, _ptr(input_global_scale), _ptr(packed), _ptr(scales),
                                          _stream_of(x, stream)))
    return packed, scales


def nvfp4_w4a4_gemm(x_packed: torch.Tensor, x_scales: torch.Tensor, input_global_scale: torch.Tensor,
                    packed: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                    bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 [M, N] = alpha * (NVFP4 x) . (NVFP4 W)^T (+ bias), alpha = gs_in * gs_w."""
    if x_packed.dim() != 2 or packed.dim() != 2 or x_packed.shape[1] != packed.shape[1]:
        raise ValueError(f"x_packed {tuple(x_packed.shape)} and packed {tuple(packed.shape)} do not match")
    m, k = x_packed.shape[0], x_packed.shape[1] * 2
    n = packed.shape[0]
    dev = packed.device
    _check_out(x_packed, (m, k // 2), (torch.uint8,), dev, "x_packed")
    _check_out(x_scales, (m, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "x_scales")
    _check_out(packed, (n, k // 2), (torch.uint8,), dev, "packed")
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "scales")
    for t, what in ((input_global_scale, "input_global_scale"), (global_scale, "global_scale")):
        if t.numel() != 1 or t.dtype != torch.float32 or t.device != dev:
            raise ValueError(f"{what} must be one float32 on the weight's device")
    if bias is not None:
        _check_out(bias, (n,), (torch.bfloat16,), dev, "bias")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, (m, n), (torch.bfloat16,), dev, "out")
    lib = load_library()
    need = int(lib.nvfp4_w4a4_workspace_bytes(m, k))
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError(f"workspace needs {need} bytes on {dev}")
    _check("nvfp4_w4a4_gemm",
           lib.nvfp4_w4a4_gemm(_ptr(x_packed), _ptr(x_scales), _ptr(input_global_scale), m, k, _ptr(packed),
                               _ptr(scales), _ptr(global_scale), n, _ptr(bias), _ptr(workspace), _ptr(out),
                               _stream_of(packed, stream)))
    return out


#: Bytes of the static scratch nvfp4_w4a4_gemm_noalloc uses (NVFP4_W4A4_SCRATCH_BYTES).
W4A4_SCRATCH_BYTES = 4 << 20


def nvfp4_w4a4_gemm_noalloc(x_packed: torch.Tensor, x_scales: torch.Tensor, input_global_scale: torch.Tensor,
                            packed: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                            out: torch.Tensor, bias: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_w4a4_gemm with the library's static scratch as workspace: the caller
    passes the output buffer and nothing is allocated (M*K <= 2097144)."""
    if x_packed.dim() != 2 or packed.dim() != 2 or x_packed.shape[1] != packed.shape[1]:
        raise ValueError(f"x_packed {tuple(x_packed.shape)} and packed {tuple(packed.shape)} do not match")
    m, k = x_packed.shape[0], x_packed.shape[1] * 2
    n = packed.shape[0]
    dev = packed.device
    _check_out(x_packed, (m, k // 2), (torch.uint8,), dev, "x_packed")
    _check_out(x_scales, (m, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "x_scales")
    _check_out(packed, (n, k // 2), (torch.uint8,), dev, "packed")
    _check_out(scales, (n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, "scales")
    for t, what in ((input_global_scale, "input_global_scale"), (global_scale, "global_scale")):
        if t.numel() != 1 or t.dtype != torch.float32 or t.device != dev:
            raise ValueError(f"{what} must be one float32 on the weight's device")
    if bias is not None:
        _check_out(bias, (n,), (torch.bfloat16,), dev, "bias")
    _check_out(out, (m, n), (torch.bfloat16,), dev, "out")
    lib = load_library()
    _check("nvfp4_w4a4_gemm_noalloc",
           lib.nvfp4_w4a4_gemm_noalloc(_ptr(x_packed), _ptr(x_scales), _ptr(input_global_scale), m, k,
                                       _ptr(packed), _ptr(scales), _ptr(global_scale), n, _ptr(bias), _ptr(out),
                                       _stream_of(packed, stream)))
    return out


# ---------------------------------------------------------------------------
# Mixture of experts (W4A16)
# ---------------------------------------------------------------------------

def _check_experts(packed: torch.Tensor, scales: torch.Tensor, global_scales: torch.Tensor, k: int, dev,
                   what: str):
    if packed.dim() != 3 or packed.shape[2] * 2 != k:
        raise ValueError(f"{what} packed shape {tuple(packed.shape)} does not match K={k}")
    e, n = packed.shape[0], packed.shape[1]
    _check_out(packed, (e, n, k // 2), (torch.uint8,), dev, f"{what} packed")
    _check_out(scales, (e, n, k // 16), (torch.float8_e4m3fn, torch.uint8), dev, f"{what} scales")
    _check_out(global_scales, (e,), (torch.float32,), dev, f"{what} global_scales")
    return e, n


def _check_ids(topk_ids: torch.Tensor, dev) -> torch.Tensor:
    if topk_ids.dtype != torch.int32 or topk_ids.device != dev:
        raise ValueError("topk_ids must be int32 on the weights' device")
    return topk_ids.contiguous()


def moe_collapse_w13_scale2(w13_weight_scale_2: torch.Tensor) -> torch.Tensor:
    """The per-expert global scale of w13 from its [E, 2] checkpoint tensor: the w1
    column, with a warning when the w3 column differs (the pages keep one scale
    for the fused w1/w3 matrix).  A slice and a comparison, no arithmetic."""
    s = w13_weight_scale_2.reshape(w13_weight_scale_2.shape[0], -1)
    if s.shape[1] > 1 and not torch.equal(s[:, 0], s[:, 1]):
        import warnings
        warnings.warn("w1_weight_scale_2 differs from w3_weight_scale_2; the w1 value serves both, "
                      "which may reduce accuracy")
    return s[:, 0].contiguous()


def nvfp4_moe_w4a16_gemm(x: torch.Tensor, topk_ids: torch.Tensor, row_div: int, packed: torch.Tensor,
                         scales: torch.Tensor, global_scales: torch.Tensor, out: torch.Tensor | None = None,
                         invalid_pairs: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """Grouped expert GEMM: bf16 [P, N], row p = x[p // row_div] . deq(W[topk_ids[p]])^T."""
    x = _as_bf16_2d(x, "x")
    rows, k = x.shape
    dev = x.device
    e, n = _check_experts(packed, scales, global_scales, k, dev, "expert")
    ids = _check_ids(topk_ids, dev).reshape(-1)
    p = ids.numel()
    if out is None:
        out = torch.empty((p, n), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, (p, n), (torch.bfloat16,), dev, "out")
    if invalid_pairs is not None and (invalid_pairs.numel() != 1 or invalid_pairs.dtype != torch.int32
                                      or invalid_pairs.device != dev):
        raise ValueError("invalid_pairs must be one int32 on the device")
    lib = load_library()
    need = int(lib.nvfp4_moe_gemm_workspace_bytes(p, e))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError(f"workspace needs {need} bytes on {dev}")
    _check("nvfp4_moe_w4a16_gemm",
           lib.nvfp4_moe_w4a16_gemm(_ptr(x), rows, k, _ptr(ids), p, int(row_div), _ptr(packed), _ptr(scales),
                                    _ptr(global_scales), e, n, _ptr(workspace), _ptr(out), _ptr(invalid_pairs),
                                    _stream_of(x, stream)))
    return out


def nvfp4_moe_silu_and_mul(h: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 [P, 2I] -> bf16 [P, I]: silu(h[:, :I]) * h[:, I:]."""
    h = _as_bf16_2d(h, "h")
    p, i2 = h.shape
    if out is None:
        out = torch.empty((p, i2 // 2), dtype=torch.bfloat16, device=h.device)
    else:
        _check_out(out, (p, i2 // 2), (torch.bfloat16,), h.device, "out")
    lib = load_library()
    _check("nvfp4_moe_silu_and_mul",
           lib.nvfp4_moe_silu_and_mul(_ptr(h), p, i2 // 2, _ptr(out), _stream_of(h, stream)))
    return out


def nvfp4_moe_combine(o: torch.Tensor, topk_weights: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """bf16 [T*topk, H] with float32 weights [T, topk] -> bf16 [T, H]."""
    o = _as_bf16_2d(o, "o")
    if topk_weights.dim() != 2 or topk_weights.dtype != torch.float32 or topk_weights.device != o.device:
        raise ValueError("topk_weights must be float32 [T, topk] on o's device")
    w = topk_weights.contiguous()
    t, k = w.shape
    hdim = o.shape[1]
    if o.shape[0] != t * k:
        raise ValueError(f"o has {o.shape[0]} rows, expected T*topk = {t * k}")
    if out is None:
        out = torch.empty((t, hdim), dtype=torch.bfloat16, device=o.device)
    else:
        _check_out(out, (t, hdim), (torch.bfloat16,), o.device, "out")
    lib = load_library()
    _check("nvfp4_moe_combine",
           lib.nvfp4_moe_combine(_ptr(o), _ptr(w), t, k, hdim, _ptr(out), _stream_of(o, stream)))
    return out


def nvfp4_moe_w4a16_forward(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                            w13: tuple, w2: tuple, out: torch.Tensor | None = None,
                            invalid_pairs: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """The W4A16 expert layer: bf16 x [T, H] -> bf16 [T, H].  ``w13`` / ``w2`` =
    (packed, scales, global_scales) with shapes [E, 2I, H/2], [E, 2I, H/16], [E]
    and [E, H, I/2], [E, H, I/16], [E]."""
    x = _as_bf16_2d(x, "x")
    t, hdim = x.shape
    dev = x.device
    e, n13 = _check_experts(*w13, hdim, dev, "w13")
    if w2[0].dim() != 3:
        raise ValueError("w2 packed must be [E, H, I/2]")
    i = w2[0].shape[2] * 2
    e2, n2 = _check_experts(*w2, i, dev, "w2")
    if n13 != 2 * i or e2 != e or n2 != hdim:
        raise ValueError(f"w13 [E, {n13}, .] and w2 [{e2}, {n2}, {i // 2}] do not fit H={hdim}")
    ids = _check_ids(topk_ids, dev)
    if ids.dim() != 2 or ids.shape[0] != t:
        raise ValueError("topk_ids must be int32 [T, topk]")
    topk = ids.shape[1]
    if tuple(topk_weights.shape) != (t, topk) or topk_weights.dtype != torch.float32 or \
            topk_weights.device != dev:
        raise ValueError("topk_weights must be float32 [T, topk] on the device")
    w = topk_weights.contiguous()
    if out is None:
        out = torch.empty((t, hdim), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, (t, hdim), (torch.bfloat16,), dev, "out")
    if invalid_pairs is not None and (invalid_pairs.numel() != 1 or invalid_pairs.dtype != torch.int32
                                      or invalid_pairs.device != dev):
        raise ValueError("invalid_pairs must be one int32 on the device")
    lib = load_library()
    need = int(lib.nvfp4_moe_workspace_bytes(t, topk, e, hdim, i))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError(f"workspace needs {need} bytes on {dev}")
    _check("nvfp4_moe_w4a16_forward",
           lib.nvfp4_moe_w4a16_forward(_ptr(x), t, hdim, _ptr(ids), _ptr(w), topk, _ptr(w13[0]), _ptr(w13[1]),
                                       _ptr(w13[2]), _ptr(w2[0]), _ptr(w2[1]), _ptr(w2[2]), e, i,
                                       _ptr(workspace), _ptr(out), _ptr(invalid_pairs), _stream_of(x, stream)))
    return out
