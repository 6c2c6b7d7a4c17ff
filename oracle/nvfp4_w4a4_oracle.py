"""Plain CPU oracle for NVFP4 W4A4: activations quantized to NVFP4 at run
time with a static global input scale, then the product of the two NVFP4
operands scaled by alpha.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

Sources (cited by page title and section):

* P2 = vLLM source view of ``vllm/model_executor/layers/quantization/modelopt.py``:
  ``KNvfp4Dynamic`` (one float32 ``input_scale`` per partition on disk; the
  global input scale is their maximum, its float32 reciprocal is kept for
  quantizing; the per-16 block scales are computed at run time),
  ``maybe_fuse_global_scales`` (``alpha = input_global_scale *
  weight_global_scale``) and the ``NVFP4`` recipe (static FP4 weight, dynamic
  FP4 activation).
* P1 = vLLM API docs, ``quantization.online.lm_head``, ``_quantize_nvfp4``:
  the block-scale and code rules, shared with the weights.

Readings (also listed in the repository's design notes):

W1  The activation's block scales and codes follow the weight quantizer's
    rules (``oracle.nvfp4_oracle.quantize_rows``, readings R1-R5) with the
    static global input scale in place of the weight's amax/2688: block scale
    ``e4m3(min(fl(fl(b/6) * inv), 448))`` with ``inv = fl32(1 / gs_in)``.
W2  ``alpha = fl32(gs_in * gs_w)`` (P2 multiplies the two float32 scalars).
W3  ``y = bf16_rne(alpha * sum_k (code_x * s_x) (code_w * s_w) + bias)``:
    each ``code * s`` is exact in bf16 and each product of two is exact in
    float32, so only the accumulation order and the final rounding differ
    from the float64 reference below.
"""

from __future__ import annotations

import numpy as np

from oracle import nvfp4_oracle as O


def collapse_input_scale(input_scales: np.ndarray) -> tuple[np.float32, np.float32]:
    """P2 ``KNvfp4Dynamic.process``: (global input scale, its reciprocal)."""
    v = np.asarray(input_scales, np.float32).reshape(-1)
    gs = np.float32(v.max())
    return gs, np.float32(np.float32(1.0) / gs)


def quantize_activations(x_bits: np.ndarray, gs_in: np.float32) -> tuple[np.ndarray, np.ndarray]:
    """W1: bf16 [M, K] -> (packed [M, K/2], e4m3 scale bytes [M, K/16])."""
    return O.quantize_rows(np.asarray(x_bits, np.uint16), np.float32(gs_in))


def alpha(gs_in: np.float32, gs_w: np.float32) -> np.float32:
    """W2."""
    return np.float32(np.float32(gs_in) * np.float32(gs_w))


def block_values(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * block scale for every element (float64, exact), no global scale."""
    codes = O.unpack_codes(packed)
    vals = O.e2m1_value(codes).astype(np.float64)
    s = O.e4m3_value(scales).astype(np.float64)
    return vals * np.repeat(s, O.GROUP, axis=1)


def gemm_ref(xp, xs, wp, ws, a: np.float32, bias_bits=None) -> np.ndarray:
    """W3 in float64, before the final bf16 rounding."""
    y = (block_values(xp, xs) @ block_values(wp, ws).T) * np.float64(a)
    if bias_bits is not None:
        y = y + O.bf16_bits_to_f32(np.asarray(bias_bits, np.uint16)).astype(np.float64)[None, :]
    return y


def gemm_abs_ref(xp, xs, wp, ws, a: np.float32, bias_bits=None) -> np.ndarray:
    """alpha * sum |x w| (+ |bias|): the scale of the float32 accumulation error."""
    y = (np.abs(block_values(xp, xs)) @ np.abs(block_values(wp, ws)).T) * np.float64(a)
    if bias_bits is not None:
        y = y + np.abs(O.bf16_bits_to_f32(np.asarray(bias_bits, np.uint16)).astype(np.float64))[None, :]
    return y
