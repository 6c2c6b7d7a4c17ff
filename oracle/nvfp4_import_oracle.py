"""Plain CPU oracle for adopting a pre-quantized NVFP4 checkpoint.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What a pre-quantized checkpoint brings (cited by page title and section):

* P2 = vLLM source view of ``vllm/model_executor/layers/quantization/modelopt.py``,
  class ``KNvfp4Static``: ``create_weights`` registers the packed weight
  [N, K/2] uint8, one float32 ``weight_scale_2`` per fused output partition
  and the float8_e4m3fn ``weight_scale`` [N, K/16], the latter filled with NaN
  so that a scale the loader never wrote is detectable; ``process`` raises if
  any block scale is still NaN, warns if the partitions' ``weight_scale_2``
  values are not all the same, and keeps their maximum, unreciprocated, as
  the global scale (ModelOpt stores amax/2688, the dequantization direction).
* P3 = vLLM API docs, ``...quantization.compressed_tensors.schemes``, class
  ``CompressedTensorsW4A16Fp4``: the same packed and block-scale layout, but
  one float32 ``weight_global_scale`` per partition stored as the inverse
  (quantization direction); ``process_weights_after_loading`` turns it into
  the dequantization global scale ``1 / max(weight_global_scale)`` in float32.

Readings (also listed in the repository's design notes):

I1  "Still NaN" means a float8_e4m3fn NaN byte: 0x7F or 0xFF (the format has
    no infinities; every other byte is a finite value).
I2  "Not all the same" is judged with IEEE equality of every later
    partition's value against the first one (so a NaN among several
    partitions counts as differing; a single partition never differs).
    P2 only warns; P3 neither warns nor checks.  The adapter reports the
    condition under both conventions and leaves the reaction to the caller.
I3  The compressed-tensors reciprocal is one IEEE float32 division of 1 by the
    float32 maximum (P3's ``1 / tensor.max().to(torch.float32)``).
I4  Beyond the pages: a collapsed global scale that is not a finite number
    greater than 0 is reported, since the GEMM cannot use it.
"""

from __future__ import annotations

import numpy as np

#: Conventions of the per-partition global scales (P2, P3).
MODELOPT = "modelopt"
COMPRESSED_TENSORS = "compressed-tensors"

#: Flag bits of the adapter's report.
FLAG_SCALES_NOT_LOADED = 1
FLAG_PARTITIONS_DIFFER = 2
FLAG_BAD_GLOBAL_SCALE = 4


def e4m3_byte_is_nan(byte: int) -> bool:
    """I1: float8_e4m3fn encodes NaN as S.1111.111 and nothing else."""
    return (byte & 0x7F) == 0x7F


def scales_not_loaded(scale_bytes: np.ndarray) -> bool:
    """P2 ``KNvfp4Static.process``: some block scale still holds the NaN
    sentinel it was created with.  One byte at a time, as written."""
    flat = np.asarray(scale_bytes, dtype=np.uint8).reshape(-1)
    for b in flat.tolist():
        if e4m3_byte_is_nan(b):
            return True
    return False


def partitions_differ(partition_scales: np.ndarray) -> bool:
    """P2's warning condition under reading I2."""
    v = np.asarray(partition_scales, dtype=np.float32).reshape(-1)
    first = v[0]
    return any(not (x == first) for x in v[1:].tolist())


def collapse_global_scale(partition_scales: np.ndarray, convention: str) -> np.float32:
    """The one dequantization-direction float32 global scale the GEMM uses.

    ModelOpt (P2): the maximum of ``weight_scale_2`` as stored.
    compressed-tensors (P3, I3): ``1 / max(weight_global_scale)`` in float32.
    """
    v = np.asarray(partition_scales, dtype=np.float32).reshape(-1)
    if v.size < 1:
        raise ValueError("at least one partition scale is needed")
    # max over the partitions, written out; a NaN anywhere makes the max NaN
    # (torch's max propagates NaN)
    m = v[0]
    for x in v[1:]:
        if np.isnan(x) or np.isnan(m):
            m = np.float32(np.nan)
        elif x > m:
            m = x
    if convention == MODELOPT:
        return np.float32(m)
    if convention == COMPRESSED_TENSORS:
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            return np.float32(np.float32(1.0) / m)
    raise ValueError(f"unknown convention {convention!r}")


def bad_global_scale(gs: np.float32) -> bool:
    """I4: not a finite number greater than 0."""
    g = np.float32(gs)
    return not (np.isfinite(g) and g > 0)


def import_report(partition_scales: np.ndarray, scale_bytes: np.ndarray, convention: str):
    """(global scale, flags) for a checkpoint's partition scales and block scales."""
    gs = collapse_global_scale(partition_scales, convention)
    flags = 0
    if scales_not_loaded(scale_bytes):
        flags |= FLAG_SCALES_NOT_LOADED
    if partitions_differ(partition_scales):
        flags |= FLAG_PARTITIONS_DIFFER
    if bad_global_scale(gs):
        flags |= FLAG_BAD_GLOBAL_SCALE
    return gs, flags


def checkpoint_partition_scales(partition_gs: np.ndarray, convention: str) -> np.ndarray:
    """How each convention stores the per-partition global scales ``gs_i``
    (dequantization direction, amax_i/2688) on disk: ModelOpt as is (P2);
    compressed-tensors as the float32 inverse (P3: it stores the inverse of
    what the kernels expect)."""
    g = np.asarray(partition_gs, dtype=np.float32).reshape(-1)
    if convention == MODELOPT:
        return g.copy()
    if convention == COMPRESSED_TENSORS:
        return (np.float32(1.0) / g).astype(np.float32)
    raise ValueError(f"unknown convention {convention!r}")
