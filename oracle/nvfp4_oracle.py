"""Plain, slow CPU oracle for online NVFP4 quantization and the W4A16 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library: every step below is written out from
the pages' description of the method, in numpy, one step per line.

Sources (cited by page title and section):

* P1 = vLLM API docs, ``vllm.model_executor.layers.quantization.online.lm_head``,
  function ``_quantize_nvfp4`` and class ``_LMHeadNvfp4Method``.
* P2 = vLLM source view of ``vllm/model_executor/layers/quantization/modelopt.py``,
  classes ``ModelOptNvFp4Config`` and ``KNvfp4Static``.
* P3 = vLLM API docs, ``...quantization.compressed_tensors.schemes``,
  class ``CompressedTensorsW4A16Fp4``.

Arithmetic: float32 wherever the method's decisions are taken (the pages build
the scales from ``.float()`` tensors), float64 for the GEMM reference.  Every
float32 operation is a single numpy float32 ufunc call, so each is IEEE
correctly rounded (round to nearest even).

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):

R1  ``ref_nvfp4_quant`` is not defined on the pages.  Block scale:
    ``u = min(fl(fl(b / 6) * inv_gs), 448)`` with ``b`` the block's max |w|,
    rounded to E4M3 (RNE).  Element: ``q = fl(w * fl(inv_gs / s))`` with ``s``
    the *stored* (rounded) scale, so that dequantization reconstructs ``w``.
R2  E2M1 rounding is round-to-nearest, ties to the even code, saturating at 6.
R3  E4M3 rounding is round-to-nearest-even (the cast P1 applies), after the
    clamp to the format maximum 448 (P1's ``fp8_max``).
R4  A block whose stored scale is 0 (all-zero block, or ``u <= 2**-10``)
    encodes every element as code 0 (no 0 * inf).
R5  The sign bit is set only when the value is strictly negative and its
    magnitude code is nonzero (P1 tests ``values < 0``; -0.0 is not < 0 and a
    value rounded to 0 has no sign), so zero is always code 0x0.
R6  ``weight_amax`` is the max |w| over the whole tensor passed in.
R7  K must be a positive multiple of 16 (P2 ``KNvfp4Static`` raises otherwise);
    non-finite weights are outside the contract and raise here.
R8  The optional bias is added to the fp64 sum (the GEMM reference), as the
    kernel adds it in fp32 before its one rounding to bf16.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Format constants (P1 ``_quantize_nvfp4``; P2 ``KNvfp4Static`` comment that the
# kernels expect the raw amax/2688 global scale).
# ---------------------------------------------------------------------------

#: Block (group) size along K: P2 ``ModelOptNvFp4Config`` default group_size,
#: P3 ``CompressedTensorsW4A16Fp4.group_size``.
GROUP = 16
#: Largest E2M1 magnitude (the top of P1's doubled-magnitude table, 12 / 2).
E2M1_MAX = 6.0
#: Largest finite float8_e4m3fn value (P1 ``torch.finfo(torch.float8_e4m3fn).max``).
E4M3_MAX = 448.0
#: Divisor of the global scale: E2M1_MAX * E4M3_MAX = 2688 (P2 "amax/2688").
GS_DIVISOR = E2M1_MAX * E4M3_MAX
#: E2M1 magnitudes by 3-bit code (P1's table maps doubled magnitudes
#: 0,1,2,3,4,6,8,12 to codes 0..7).
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

F32 = np.float32


class OracleContractError(ValueError):
    """Input outside the method's contract (R7)."""


# ---------------------------------------------------------------------------
# bf16 / e4m3 / e2m1 value helpers
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly equal float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """float8_e4m3fn byte -> value (float64), from the format definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    is subnormal with step 2**-9; 0x7F/0xFF are NaN; there is no infinity.
    """
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode_rne(u: np.ndarray) -> np.ndarray:
    """Non-negative float32 ``u`` (already clamped to <= 448) -> e4m3fn byte.

    Round to nearest, ties to the even mantissa (reading R3).  Works in float64,
    where every step below is exact for float32 inputs.
    """
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    if np.any(u < 0) or np.any(u > E4M3_MAX) or not np.all(np.isfinite(u)):
        raise OracleContractError("e4m3_encode_rne expects 0 <= u <= 448")
    out = np.zeros(u.shape, dtype=np.int64)
    sub = u < 2.0 ** -6
    # Subnormal range: value = m * 2**-9, m in 0..8 (m == 8 is the smallest
    # normal, 2**-6, whose byte is also 8).
    out[sub] = np.rint(u[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    mant, exp = np.frexp(u[nrm])          # u = mant * 2**exp, mant in [0.5, 1)
    e = exp - 1                           # u = (2*mant) * 2**e, 2*mant in [1, 2)
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # 0..8, RNE
    # m == 8 carries into the exponent; the byte arithmetic absorbs it.
    out[nrm] = ((e + 7) << 3) + m
    return out.astype(np.uint8)


def e2m1_magnitude_code(a: np.ndarray) -> np.ndarray:
    """Magnitude ``0 <= a <= 6`` (float32) -> 3-bit E2M1 code (reading R2).

    Nearest grid point; a value exactly between two grid points goes to the
    even code.  The midpoints of consecutive grid values are
    0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; the even code wins each tie, so the
    lower neighbour wins at 0.25, 1.25, 2.5 and 5 and the upper at 0.75, 1.75
    and 3.5.
    """
    a = np.asarray(a, dtype=np.float32)
    code = np.zeros(a.shape, dtype=np.uint8)
    code += (a > F32(0.25))
    code += (a >= F32(0.75))
    code += (a > F32(1.25))
    code += (a >= F32(1.75))
    code += (a > F32(2.5))
    code += (a >= F32(3.5))
    code += (a > F32(5.0))
    return code


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """4-bit code (bit 3 = sign, P1) -> value (float64)."""
    c = np.asarray(code, dtype=np.uint8)
    grid = np.asarray(E2M1_GRID, dtype=np.float64)
    mag = grid[c & 0x7]
    return np.where(c & 0x8, -mag, mag)


# ---------------------------------------------------------------------------
# Quantization: P1 ``_quantize_nvfp4`` (global scale, block scales, codes,
# packing), with the readings R1-R7.
# ---------------------------------------------------------------------------

def check_weight(w_bits: np.ndarray) -> tuple[int, int]:
    w_bits = np.asarray(w_bits)
    if w_bits.dtype != np.uint16 or w_bits.ndim != 2:
        raise OracleContractError("weight must be a 2-D array of bf16 bits (uint16)")
    n, k = w_bits.shape
    if n < 1 or k < GROUP or k % GROUP != 0:
        raise OracleContractError(f"need N >= 1 and K a positive multiple of {GROUP}; got {n}x{k}")
    if np.any((w_bits & 0x7F80) == 0x7F80):
        raise OracleContractError("non-finite weight")
    return n, k


def weight_amax(w_bits: np.ndarray, chunk_rows: int = 4096) -> np.float32:
    """Max |w| over the whole tensor (reading R6).  Exact: a max of bf16 values."""
    best = F32(0.0)
    for r0 in range(0, w_bits.shape[0], chunk_rows):
        best = max(best, F32(np.max(np.abs(bf16_bits_to_f32(w_bits[r0:r0 + chunk_rows])))))
    return best


def global_scale(amax: np.float32) -> np.float32:
    """Dequantization-direction global scale (P1 ``_quantize_nvfp4``).

    ``gs = max(fl32(amax / (6 * 448)), fl32(1e-12))``; the clamp constant is the
    Python float 1e-12 applied to a float32 tensor, i.e. fl32(1e-12).
    """
    gs = F32(amax) / F32(GS_DIVISOR)
    return max(F32(gs), F32(1e-12))


def inverse_global_scale(gs: np.float32) -> np.float32:
    """``fl32(1 / gs)`` (P1 ``_quantize_nvfp4``: ``1.0 / global_scale``)."""
    return F32(1.0) / F32(gs)


def block_scales(w_rows_f32: np.ndarray, inv_gs: np.float32) -> tuple[np.ndarray, np.ndarray]:
    """Per-16 block scales (reading R1), for float32 rows ``[n, K]``.

    Returns the e4m3fn bytes ``[n, K/16]`` and their values as float32.
    """
    n, k = w_rows_f32.shape
    blocks = np.abs(w_rows_f32.reshape(n, k // GROUP, GROUP))
    b = blocks.max(axis=2).astype(np.float32)          # block max |w|
    t = b / F32(E2M1_MAX)                              # fl32(b / 6)
    u = t * F32(inv_gs)                                # fl32(t * inv_gs)
    u = np.minimum(u, F32(E4M3_MAX))                   # clamp to fp8 max
    s_bytes = e4m3_encode_rne(u)
    s_vals = e4m3_value(s_bytes).astype(np.float32)    # exact in float32
    return s_bytes, s_vals


def element_codes(w_rows_f32: np.ndarray, s_vals: np.ndarray, inv_gs: np.float32) -> np.ndarray:
    """4-bit codes ``[n, K]`` for float32 rows, given the stored block scales."""
    n, k = w_rows_f32.shape
    safe = np.where(s_vals > 0, s_vals, F32(1.0)).astype(np.float32)
    r = np.where(s_vals > 0, F32(inv_gs) / safe, F32(0.0)).astype(np.float32)   # fl32(inv / s)
    q = w_rows_f32.reshape(n, k // GROUP, GROUP) * r[:, :, None]               # fl32(w * r)
    q = q.astype(np.float32).reshape(n, k)
    a = np.minimum(np.abs(q), F32(E2M1_MAX))
    mag = e2m1_magnitude_code(a)
    neg = (q < 0) & (mag != 0)
    return (mag | (neg.astype(np.uint8) << 3)).astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, the even-k code in the low nibble (P1)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n, h = packed.shape
    out = np.empty((n, 2 * h), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize_rows(w_bits_rows: np.ndarray, gs: np.float32) -> tuple[np.ndarray, np.ndarray]:
    """Quantize some rows given the tensor's global scale: (packed, scale bytes).

    Every step after the global scale is row-local, so a row subset of a large
    tensor quantizes to exactly its rows of the full result.
    """
    w = bf16_bits_to_f32(w_bits_rows)
    inv = inverse_global_scale(gs)
    s_bytes, s_vals = block_scales(w, inv)
    codes = element_codes(w, s_vals, inv)
    return pack_codes(codes), s_bytes


def quantize(w_bits: np.ndarray, chunk_rows: int = 4096) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Full quantization: (packed u8 [N, K/2], scales u8 [N, K/16], gs float32)."""
    n, k = check_weight(w_bits)
    gs = global_scale(weight_amax(w_bits))
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // GROUP), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        p, s = quantize_rows(w_bits[r0:r0 + chunk_rows], gs)
        packed[r0:r0 + chunk_rows] = p
        scales[r0:r0 + chunk_rows] = s
    return packed, scales, gs


# ---------------------------------------------------------------------------
# Dequantization and the GEMM reference (P1 ``_LMHeadNvfp4Method.apply``:
# activations stay in the model dtype; logits = x . W^T (+ bias)).
# ---------------------------------------------------------------------------

def dequantize(packed: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    """``w_deq[n, k] = D(code) * value(scale[n, k // 16]) * gs`` in float64 (exact)."""
    codes = unpack_codes(packed)
    n, k = codes.shape
    d = e2m1_value(codes).reshape(n, k // GROUP, GROUP)
    s = e4m3_value(scales)[:, :, None]
    return (d * s).reshape(n, k) * float(gs)


def gemm_ref(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, gs: float,
             bias_bits: np.ndarray | None = None, chunk_rows: int = 8192) -> np.ndarray:
    """fp64 logits ``y[m, n] = sum_k x[m, k] * w_deq[n, k] (+ bias[n])``."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    n = packed.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        wd = dequantize(packed[r0:r0 + chunk_rows], scales[r0:r0 + chunk_rows], gs)
        y[:, r0:r0 + chunk_rows] = x @ wd.T
    if bias_bits is not None:
        y += bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return y


def gemm_tolerance(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, gs: float,
                   rtol: float = 1e-3, bias_bits: np.ndarray | None = None,
                   chunk_rows: int = 8192) -> np.ndarray:
    """Per-element bound ``rtol * ||x_m||_2 * ||w_deq_n||_2`` (+ 2**-8 |bias_n|)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    xn = np.linalg.norm(x, axis=1)
    n = packed.shape[0]
    wn = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        wd = dequantize(packed[r0:r0 + chunk_rows], scales[r0:r0 + chunk_rows], gs)
        wn[r0:r0 + chunk_rows] = np.linalg.norm(wd, axis=1)
    tol = rtol * xn[:, None] * wn[None, :]
    if bias_bits is not None:
        tol = tol + 2.0 ** -8 * np.abs(bf16_bits_to_f32(bias_bits).astype(np.float64))[None, :]
    return tol


def gemm_ref_with_norms(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, gs: float,
                        bias_bits: np.ndarray | None = None, chunk_rows: int = 8192):
    """One pass over the weight rows giving what a parity check needs.

    Returns ``(y64, w_norm, abs_sum)``: the fp64 logits of ``gemm_ref``, the
    2-norm of every dequantized weight row, and ``sum_k |x[m,k]| |w_deq[n,k]|``
    (the magnitude that bounds any fp32 summation error).
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    xa = np.abs(x)
    n = packed.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    s_abs = np.empty((x.shape[0], n), dtype=np.float64)
    wn = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        wd = dequantize(packed[r0:r0 + chunk_rows], scales[r0:r0 + chunk_rows], gs)
        y[:, r0:r0 + chunk_rows] = x @ wd.T
        s_abs[:, r0:r0 + chunk_rows] = xa @ np.abs(wd).T
        wn[r0:r0 + chunk_rows] = np.linalg.norm(wd, axis=1)
    if bias_bits is not None:
        y += bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return y, wn, s_abs


def bf16_round_rne(y: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even) as float64, via exact float32 steps.

    Used only by the one-hot closed form, where ``y`` is already a float32 value.
    """
    f = np.asarray(y, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def argmax_agreement(y_bf16: np.ndarray, y64: np.ndarray) -> tuple[float, float]:
    """(tie-aware rate, strict rate) of per-row argmax agreement.

    Tie-aware: a row passes when the fp64 winner's bf16 logit equals the row's
    bf16 maximum, i.e. the exact winner is among the rows' tied maxima.
    """
    y_bf16 = np.asarray(y_bf16, dtype=np.float64)
    win64 = np.argmax(y64, axis=1)
    rows = np.arange(y64.shape[0])
    tie_ok = y_bf16[rows, win64] == y_bf16.max(axis=1)
    strict = np.argmax(y_bf16, axis=1) == win64
    return float(tie_ok.mean()), float(strict.mean())
