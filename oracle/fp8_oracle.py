"""Plain CPU oracle for the FP8 lm_head copy (per-row weight scales,
per-token dynamic activation scales, scaled FP8 GEMM).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

Sources (cited by page title and section):

* P1 = vLLM API docs, ``vllm.model_executor.layers.quantization.online.lm_head``,
  ``quantized_lm_head_copy``: the "fp8" copy uses per-row weight scales and
  per-token activation scales on an FP8 linear kernel.
* P2 = vLLM source view of ``vllm/model_executor/layers/quantization/modelopt.py``:
  ``KFp8StaticChannel`` (weight float8_e4m3fn [N, K] with one float32 scale
  per output row) and the ``FP8_PER_CHANNEL_PER_TOKEN`` recipe (per-channel
  static weight, dynamic per-token activation).
* P3 = vLLM API docs, ``...quantization.compressed_tensors.schemes``: the W8A8
  FP8 ``apply_weights`` path, which quantizes the input per token
  (``scaled_fp8_quant(x, use_per_token_if_dynamic=True)``) and calls a scaled
  matmul with ``scale_a`` (per token), ``scale_b`` (per output channel), the
  input's dtype as output dtype and the bias.

The pages never show the quantizer's arithmetic.  Readings (also listed in
the repository's design notes):

F1  Row scale: ``s = max(fl32(amax_row / 448), fl32(1e-12))`` with 448 the
    largest float8_e4m3fn value; the clamp mirrors P1's NVFP4 global-scale
    clamp, so an all-zero row gets a finite scale and codes 0.
F2  Element: ``q = e4m3_rne(clamp(fl32(x * fl32(1 / s)), -448, 448))``: one
    reciprocal per row and a multiply per element (the pattern P1's NVFP4
    quantizer uses with its inverse global scale), saturating at 448,
    round to nearest even, the sign kept (-0.0 becomes 0x80).
F3  The same row rule serves the weight (per output row, once) and the
    activations (per token, at every call).
F4  GEMM: ``y[m, n] = bf16_rne(s_x[m] * s_w[n] * sum_k e4m3(xq[m,k]) *
    e4m3(wq[n,k]) + bias[n])``; each product of two e4m3 values is exact in
    float32, the accumulation is float32 in the kernel and float64 here.
"""

from __future__ import annotations

import numpy as np

from oracle import nvfp4_oracle as O

#: Largest finite float8_e4m3fn value (P1 ``torch.finfo(torch.float8_e4m3fn).max``).
E4M3_MAX = np.float32(448.0)
#: Smallest row scale (F1, the clamp P1 applies to the NVFP4 global scale).
SCALE_MIN = np.float32(1e-12)


def e4m3_encode_signed(v: np.ndarray) -> np.ndarray:
    """float32 values with |v| <= 448 -> float8_e4m3fn bytes, RNE, sign kept.
    The magnitude goes through the NVFP4 oracle's E4M3 encoder (written out
    from the format's definition and pinned there)."""
    v = np.asarray(v, dtype=np.float32)
    mag = O.e4m3_encode_rne(np.abs(v)).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e4m3_decode_signed(code: np.ndarray) -> np.ndarray:
    """float8_e4m3fn bytes -> float64 values (finite codes only)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = O.e4m3_value(code & 0x7F).astype(np.float64)
    return np.where(code & 0x80, -mag, mag)


def row_scale(amax: np.float32) -> tuple[np.float32, np.float32]:
    """F1: (s, 1/s) of a row with largest magnitude ``amax``."""
    s = np.float32(np.float32(amax) / E4M3_MAX)
    if s < SCALE_MIN:
        s = SCALE_MIN
    inv = np.float32(np.float32(1.0) / s)
    return s, inv


def quantize_rows(a_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [R, K] -> (float8_e4m3fn bytes [R, K], float32 scales [R])."""
    a = O.bf16_bits_to_f32(np.asarray(a_bits, dtype=np.uint16))
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input")
    r, k = a.shape
    q = np.empty((r, k), np.uint8)
    scales = np.empty(r, np.float32)
    for i in range(r):
        amax = np.float32(np.abs(a[i]).max()) if k else np.float32(0)
        s, inv = row_scale(amax)
        v = (a[i] * inv).astype(np.float32)                     # one float32 multiply per element
        v = np.minimum(np.maximum(v, -E4M3_MAX), E4M3_MAX)       # saturate (F2)
        q[i] = e4m3_encode_signed(v)
        scales[i] = s
    return q, scales


def gemm_ref(xq: np.ndarray, xs: np.ndarray, wq: np.ndarray, ws: np.ndarray,
             bias_bits: np.ndarray | None = None) -> np.ndarray:
    """F4 in float64: [M, N] logits before the final bf16 rounding."""
    xv = e4m3_decode_signed(xq)
    wv = e4m3_decode_signed(wq)
    acc = xv @ wv.T
    y = acc * np.asarray(xs, np.float64)[:, None] * np.asarray(ws, np.float64)[None, :]
    if bias_bits is not None:
        y = y + O.bf16_bits_to_f32(np.asarray(bias_bits, np.uint16)).astype(np.float64)[None, :]
    return y


def gemm_abs_ref(xq, xs, wq, ws, bias_bits=None) -> np.ndarray:
    """sum_k |x w| * s_x * s_w (+ |bias|): the scale of the float32
    accumulation error."""
    xv = np.abs(e4m3_decode_signed(xq))
    wv = np.abs(e4m3_decode_signed(wq))
    y = (xv @ wv.T) * np.asarray(xs, np.float64)[:, None] * np.asarray(ws, np.float64)[None, :]
    if bias_bits is not None:
        y = y + np.abs(O.bf16_bits_to_f32(np.asarray(bias_bits, np.uint16)).astype(np.float64))[None, :]
    return y
