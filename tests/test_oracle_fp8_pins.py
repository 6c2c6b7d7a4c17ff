"""Pins of the FP8 oracle (oracle/fp8_oracle.py) against independent
definitions: torch's own float8_e4m3fn casts, closed forms of the row-scale
rule, exact rational sums for the GEMM, and properties every row must have."""

import fractions

import numpy as np
import pytest
import torch

import oracle.fp8_oracle as F
from nvfp4_w4a16_lm_amd import workloads as wl


def torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_for_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    got = F.e4m3_decode_signed(codes)
    assert np.array_equal(got, want)


def test_encode_matches_torch_cast_on_random_and_tie_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),             # subnormal range
        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties go to the even mantissa)
    vals = F.e4m3_decode_signed(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    assert np.array_equal(F.e4m3_encode_signed(v), torch_e4m3(v))


def test_row_scale_closed_forms():
    assert F.row_scale(np.float32(448.0)) == (np.float32(1.0), np.float32(1.0))
    assert F.row_scale(np.float32(0.0))[0] == np.float32(1e-12)
    s, inv = F.row_scale(np.float32(7.0))
    assert s == np.float32(7.0) / np.float32(448.0) and inv == np.float32(1.0) / s


def test_quantize_rows_matches_a_torch_pipeline():
    """The same reading written with torch ops (independent arithmetic)."""
    rng = np.random.default_rng(2)
    bits = wl.random_weight_bits(37, 96, sigma=0.05, seed=3)
    bits[5] = 0                                             # an all-zero row
    q, s = F.quantize_rows(bits)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    ts = (x.abs().amax(dim=1) / 448.0).clamp(min=np.float32(1e-12))
    tq = (x * (1.0 / ts)[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, ts.numpy())
    assert np.array_equal(q, tq)


def test_row_maximum_maps_to_448_and_zero_rows_to_zero():
    bits = wl.random_weight_bits(64, 128, sigma=0.02, seed=9)
    bits[3] = 0
    q, s = F.quantize_rows(bits)
    a = wl.bf16_bits_to_f32(bits)
    for i in range(64):
        if i == 3:
            assert not q[i].any() and s[i] == np.float32(1e-12)
            continue
        j = int(np.argmax(np.abs(a[i])))
        assert q[i, j] & 0x7F == 0x7E
        # reconstruction within half a code step (relative 2^-4) plus the subnormal step
        err = np.abs(F.e4m3_decode_signed(q[i]) * s[i] - a[i])
        assert np.all(err <= np.abs(a[i]) * 2.0 ** -4 + s[i] * 2.0 ** -10 + 1e-30)


def test_negative_zero_keeps_its_sign():
    bits = np.zeros((1, 16), np.uint16)
    bits[0, 0] = 0x8000            # -0.0
    bits[0, 1] = 0x3F80            # 1.0
    q, _ = F.quantize_rows(bits)
    assert q[0, 0] == 0x80 and q[0, 1] == 0x7E and not q[0, 2:].any()


def test_gemm_ref_is_the_exact_rational_sum():
    rng = np.random.default_rng(4)
    # codes with exponents in a narrow band so every float64 sum is exact
    pool = np.array([c for c in range(0x30, 0x50)] + [c | 0x80 for c in range(0x30, 0x50)], np.uint8)
    xq = rng.choice(pool, (3, 32))
    wq = rng.choice(pool, (5, 32))
    xs = np.float32([0.5, 0.25, 2.0])
    ws = np.float32([1.0, 0.125, 4.0, 0.5, 8.0])
    y = F.gemm_ref(xq, xs, wq, ws)
    for m in range(3):
        for n in range(5):
            tot = sum(fractions.Fraction(float(F.e4m3_decode_signed(xq[m, k]))) *
                      fractions.Fraction(float(F.e4m3_decode_signed(wq[n, k]))) for k in range(32))
            assert y[m, n] == float(tot * fractions.Fraction(float(xs[m])) * fractions.Fraction(float(ws[n])))


def test_gemm_ref_bias_is_added():
    xq = np.full((2, 16), 0x38, np.uint8)                  # 1.0
    wq = np.full((3, 16), 0x40, np.uint8)                  # 2.0
    bias = np.array([0x3F80, 0xBF80, 0x0000], np.uint16)   # 1, -1, 0
    y = F.gemm_ref(xq, np.float32([1, 1]), wq, np.float32([1, 1, 1]), bias)
    assert np.array_equal(y, np.array([[33.0, 31.0, 32.0]] * 2))
