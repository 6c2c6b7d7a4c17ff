"""NVFP4 W4A16 lm_head for MI355X (gfx950): online quantization + W4A16 GEMM.

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libnvfp4_w4a16.so``, declared in ``include/nvfp4_w4a16.h``).  This package is
its thin ctypes binding; it loads the library on first use of an entry point and
raises if the library is missing (there is no fallback path).
"""

_API = ("nvfp4_quantize", "nvfp4_refresh_inplace", "nvfp4_w4a16_gemm", "NVFP4ShapeError",
        "NVFP4Error", "library_path", "load_library", "STATUS_NAMES")


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_API)
