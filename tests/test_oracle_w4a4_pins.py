"""Pins of the W4A4 oracle (oracle/nvfp4_w4a4_oracle.py): the pages' scalar
expressions evaluated by torch, the link to the (pinned) weight quantizer,
exact round trips of activations already on the NVFP4 grid, and exact
rational sums for the GEMM reference."""

import fractions

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import workloads as wl


def test_collapse_input_scale_is_torch_max_and_reciprocal():
    v = np.float32([3e-3, 7e-3, 5e-3])
    gs, inv = A.collapse_input_scale(v)
    t = torch.from_numpy(v).max().to(torch.float32)
    assert gs == np.float32(t.item()) and inv == np.float32((1.0 / t).to(torch.float32).item())


def test_alpha_is_the_float32_product():
    rng = np.random.default_rng(0)
    for _ in range(50):
        a, b = np.float32(rng.uniform(1e-5, 1e-1)), np.float32(rng.uniform(1e-5, 1e-1))
        assert A.alpha(a, b) == np.float32((torch.tensor(a) * torch.tensor(b)).item())
    assert A.alpha(np.float32(2.0 ** -7), np.float32(2.0 ** -9)) == np.float32(2.0 ** -16)


def test_own_global_scale_reproduces_the_weight_quantizer():
    x = wl.random_activation_bits(9, 96, seed=4)
    p, s, gs = O.quantize(x)
    ap, as_ = A.quantize_activations(x, gs)
    assert np.array_equal(ap, p) and np.array_equal(as_, s)


def test_grid_values_round_trip_exactly():
    """x = code * s * gs_in with gs_in a power of two and each block holding
    +-6 * s: the quantizer returns the same codes and scale bytes."""
    rng = np.random.default_rng(5)
    gs_in = np.float32(2.0 ** -6)
    m, k = 4, 64
    sbytes = rng.integers(0x20, 0x60, size=(m, k // 16)).astype(np.uint8)
    codes = rng.integers(0, 16, size=(m, k)).astype(np.uint8)
    codes[:, ::16] = 7                                # +6 in every block fixes its scale
    codes[(codes & 7) == 0] = 0                        # no -0 codes
    vals = O.e2m1_value(codes) * np.repeat(O.e4m3_value(sbytes), 16, axis=1) * float(gs_in)
    x = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.float().numpy(), vals.astype(np.float32))   # exact in bf16
    xb = x.view(torch.int16).numpy().view(np.uint16)
    p, s = A.quantize_activations(xb, gs_in)
    assert np.array_equal(s, sbytes)
    assert np.array_equal(O.unpack_codes(p), codes)


def test_gemm_ref_is_the_exact_rational_sum():
    rng = np.random.default_rng(6)
    x = wl.random_activation_bits(3, 32, seed=1)
    w = wl.random_weight_bits(4, 32, seed=2)
    wp, ws, gw = O.quantize(w)
    gi = np.float32(2.0 ** -8)
    xp, xs = A.quantize_activations(x, gi)
    a = A.alpha(gi, gw)
    y = A.gemm_ref(xp, xs, wp, ws, a)
    xv, wv = A.block_values(xp, xs), A.block_values(wp, ws)
    for i in range(3):
        for j in range(4):
            tot = sum(fractions.Fraction(float(xv[i, k])) * fractions.Fraction(float(wv[j, k])) for k in range(32))
            want = float(tot * fractions.Fraction(float(a)))
            assert abs(y[i, j] - want) <= 2.0 ** -50 * abs(want)
