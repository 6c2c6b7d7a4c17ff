"""Pins of the checkpoint-import oracle (oracle/nvfp4_import_oracle.py) against
what the pages and independent library routines fix.

* NaN sentinel: torch's own float8_e4m3fn decoding says which bytes are NaN
  (vLLM modelopt.py, KNvfp4Static.process tests ``torch.isnan`` of the scales).
* Global scales: the pages' expressions evaluated by torch on the CPU
  (``weight_scale_2.max()`` for ModelOpt; ``1 / weight_global_scale.max()`` in
  float32 for compressed-tensors), an exact rational rounding of 1/m to
  float32, closed forms for powers of two, and the round trip of a global
  scale produced by the quantization oracle.
* The "partitions differ" condition: ``torch.unique(...).numel() != 1``.
"""

import fractions
import struct

import numpy as np
import pytest
import torch

import oracle.nvfp4_import_oracle as I
import oracle.nvfp4_oracle as O


def test_e4m3_nan_bytes_match_torch_decoding():
    allb = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    want = torch.isnan(allb).tolist()
    got = [I.e4m3_byte_is_nan(b) for b in range(256)]
    assert got == want
    assert [b for b in range(256) if got[b]] == [0x7F, 0xFF]


@pytest.mark.parametrize("pos", ["first", "middle", "last"])
@pytest.mark.parametrize("nan_byte", [0x7F, 0xFF])
def test_scales_not_loaded_finds_one_sentinel(pos, nan_byte):
    rng = np.random.default_rng(3)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    s = rng.choice(finite, size=(7, 33))
    assert not I.scales_not_loaded(s)
    i = {"first": 0, "middle": s.size // 2, "last": s.size - 1}[pos]
    s.reshape(-1)[i] = nan_byte
    assert I.scales_not_loaded(s)
    assert I.scales_not_loaded(s) == bool(torch.isnan(torch.from_numpy(s).view(torch.float8_e4m3fn).float()).any())


def test_every_finite_byte_counts_as_loaded():
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    assert finite.size == 254
    assert not I.scales_not_loaded(finite)
    assert I.scales_not_loaded(np.full((4, 4), 0x7F, np.uint8))   # a fresh sentinel-filled buffer


def _f32(v):
    return np.asarray(v, dtype=np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_modelopt_collapse_is_torch_max(seed):
    rng = np.random.default_rng(seed)
    v = _f32(rng.uniform(1e-6, 1e-2, size=1 + seed))
    want = torch.from_numpy(v).max().to(torch.float32).item()
    assert I.collapse_global_scale(v, I.MODELOPT) == np.float32(want)


@pytest.mark.parametrize("seed", range(6))
def test_compressed_tensors_collapse_is_torch_reciprocal_of_max(seed):
    rng = np.random.default_rng(100 + seed)
    v = _f32(rng.uniform(10.0, 1e5, size=1 + seed))
    want = (1 / torch.from_numpy(v).max().to(torch.float32)).item()
    got = I.collapse_global_scale(v, I.COMPRESSED_TENSORS)
    assert got.dtype == np.float32 and np.float32(want) == got


def _round_to_f32_exact(q: fractions.Fraction) -> np.float32:
    """Nearest-even float32 of a positive rational in the normal range, from its bits."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while fractions.Fraction(2) ** e > q:
        e -= 1
    while fractions.Fraction(2) ** (e + 1) <= q:
        e += 1
    assert -126 <= e <= 127
    scaled = q / fractions.Fraction(2) ** (e - 23)        # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > fractions.Fraction(1, 2) or (rem == fractions.Fraction(1, 2) and m % 2 == 1):
        m += 1
    if m == 1 << 24:
        m, e = 1 << 23, e + 1
    bits = ((e + 127) << 23) | (m - (1 << 23))
    return np.float32(struct.unpack("<f", struct.pack("<I", bits))[0])


@pytest.mark.parametrize("seed", range(20))
def test_compressed_tensors_reciprocal_is_correctly_rounded(seed):
    rng = np.random.default_rng(200 + seed)
    m = np.float32(rng.uniform(1.0, 1e6))
    got = I.collapse_global_scale(_f32([m]), I.COMPRESSED_TENSORS)
    assert got == _round_to_f32_exact(fractions.Fraction(1) / fractions.Fraction(float(m)))


@pytest.mark.parametrize("e", [-20, -3, 0, 5, 30])
def test_powers_of_two_are_exact_both_ways(e):
    g = np.float32(2.0 ** e)
    for conv in (I.MODELOPT, I.COMPRESSED_TENSORS):
        stored = I.checkpoint_partition_scales(_f32([g]), conv)
        assert I.collapse_global_scale(stored, conv) == g


def test_round_trip_of_an_oracle_global_scale():
    # a bf16 amax (an exact bf16 value, as the quantization oracle sees one)
    gs = O.global_scale(np.float32(O.bf16_bits_to_f32(np.array([0x3D95], np.uint16))[0]))
    assert I.collapse_global_scale(I.checkpoint_partition_scales(_f32([gs]), I.MODELOPT), I.MODELOPT) == gs
    back = I.collapse_global_scale(I.checkpoint_partition_scales(_f32([gs]), I.COMPRESSED_TENSORS),
                                   I.COMPRESSED_TENSORS)
    # two correctly rounded reciprocals: within one unit in the last place
    assert abs(int(np.float32(back).view(np.uint32)) - int(np.float32(gs).view(np.uint32))) <= 1


@pytest.mark.parametrize("vals", [[1.0], [1.0, 1.0, 1.0], [1.0, 1.0, 2.0], [2.0, 1.0],
                                  [float("nan")], [float("nan"), float("nan")], [1.0, float("nan")],
                                  [0.0, -0.0]])
def test_partitions_differ_matches_torch_unique(vals):
    v = _f32(vals)
    want = torch.unique(torch.from_numpy(v)).numel() != 1
    assert I.partitions_differ(v) == want


def test_nan_partition_scale_propagates_like_torch_max():
    v = _f32([1e-3, float("nan"), 2e-3])
    assert np.isnan(torch.from_numpy(v).max().item())
    for conv in (I.MODELOPT, I.COMPRESSED_TENSORS):
        assert np.isnan(I.collapse_global_scale(v, conv))
        assert I.bad_global_scale(I.collapse_global_scale(v, conv))


@pytest.mark.parametrize("gs,bad", [(1e-3, False), (1e-12, False), (0.0, True), (-1e-3, True),
                                    (float("inf"), True), (float("nan"), True)])
def test_bad_global_scale(gs, bad):
    assert I.bad_global_scale(np.float32(gs)) == bad


def test_import_report_flags():
    s = np.zeros((3, 4), np.uint8)
    gs, f = I.import_report(_f32([1e-3]), s, I.MODELOPT)
    assert gs == np.float32(1e-3) and f == 0
    s[1, 2] = 0x7F
    _, f = I.import_report(_f32([1e-3, 2e-3]), s, I.MODELOPT)
    assert f == I.FLAG_SCALES_NOT_LOADED | I.FLAG_PARTITIONS_DIFFER
    gs, f = I.import_report(_f32([0.0]), np.zeros(1, np.uint8), I.COMPRESSED_TENSORS)
    assert np.isinf(gs) and f == I.FLAG_BAD_GLOBAL_SCALE
