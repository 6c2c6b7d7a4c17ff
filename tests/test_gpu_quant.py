"""GPU parity: nvfp4_quantize / nvfp4_refresh_inplace against the CPU oracle.

Bit-exact on packed codes, scale bytes and the global scale's fp32 bits.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import (DEV, assert_quant_equal, dev_bf16, f32_bits, quantize_gpu, upload_quant)

pytestmark = pytest.mark.gpu


def check(w_bits, label):
    got = quantize_gpu(w_bits)
    want = O.quantize(w_bits)
    assert_quant_equal(w_bits, got, want, label)


def test_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    check(wl.weight_bits(w), "tiny")


@pytest.mark.parametrize("n,k", [(1, 16), (1, 32), (3, 48), (7, 272), (16, 256), (33, 1040),
                                 (64, 4096), (129, 4112), (1000, 512), (257, 7168)])
def test_ragged_shapes(n, k):
    check(wl.random_weight_bits(n, k, sigma=0.05, seed=n), f"{n}x{k}")


@pytest.mark.parametrize("sigma", [1e-30, 1e-10, 1e-6, 1.0, 1e4, 1e30])
def test_scale_ranges(sigma):
    """Tiny amax (global-scale clamp, subnormal block scales) to huge amax."""
    check(wl.random_weight_bits(64, 256, sigma=sigma, seed=3), f"sigma={sigma}")


def test_all_zero_and_negative_zero():
    z = np.zeros((5, 64), np.uint16)
    z[2] = 0x8000
    got = quantize_gpu(z)
    assert f32_bits(got[2]) == f32_bits(np.float32(1e-12))
    assert not got[0].any() and not got[1].any()
    check(z, "zeros")


def test_zero_blocks_and_rows():
    w = wl.random_weight_bits(9, 128, sigma=0.02, seed=5)
    w[0] = 0
    w[3, 32:48] = 0
    w[4, 16:32] = 0x8000
    check(w, "zero rows/blocks")


def test_bf16_subnormal_and_extreme_values():
    w = wl.random_weight_bits(8, 64, sigma=1.0, seed=7)
    w[1] = np.arange(1, 65, dtype=np.uint16)            # positive bf16 subnormals
    w[2] = np.arange(1, 65, dtype=np.uint16) | 0x8000   # negative subnormals
    w[3, 0] = 0x7F7F                                    # largest finite bf16
    w[3, 1] = 0xFF7F
    w[4, :] = 0x0080                                    # smallest normal
    check(w, "extremes")


def test_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    w = np.array(ex["weights"], dtype=np.float64)
    for idx, val in ex["exact_weights"].items():
        if not idx.startswith("_"):
            w[int(idx)] = val[0] * 2.0 ** val[1]
    wb = wl.f32_to_bf16_bits(w.astype(np.float32))[None, :]
    p, s, g = quantize_gpu(wb)
    assert float(g) == ex["expected_gs"]
    assert s[0].tolist() == ex["expected_scales"]
    assert O.unpack_codes(p)[0].tolist() == ex["expected_codes"]


def test_grid_row_and_ties():
    """E2M1-grid rows keep their codes; E2M1 and E4M3 midpoints round to even."""
    k = 7168
    w = wl.random_weight_bits(6, k, sigma=0.01, seed=8)
    w[5] = wl.grid_row_bits(k)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    w[0, :16] = wl.f32_to_bf16_bits(np.concatenate([ties, -ties]) * np.float32(2 ** -4))
    check(w, "grid/ties")


def test_outlier_like_distribution():
    w = wl.random_weight_bits(256, 1024, sigma=0.02, seed=11)
    rng = np.random.default_rng(1)
    idx = rng.choice(w.size, 300, replace=False)
    f = wl.bf16_bits_to_f32(w).reshape(-1).copy()
    f[idx] *= 20
    check(wl.f32_to_bf16_bits(f.reshape(w.shape)), "outliers")


def test_refresh_inplace_same_pointers_and_bytes():
    w0 = wl.random_weight_bits(300, 512, sigma=0.02, seed=1)
    w1 = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(w0) + np.float32(1e-3) *
                             np.random.default_rng(2).standard_normal(w0.shape, dtype=np.float32))
    p, s, g = B.nvfp4_quantize(dev_bf16(w0))
    ptrs = (p.data_ptr(), s.data_ptr(), g.data_ptr())
    B.nvfp4_refresh_inplace(dev_bf16(w1), p, s, g)
    torch.cuda.synchronize()
    assert (p.data_ptr(), s.data_ptr(), g.data_ptr()) == ptrs
    got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
    assert_quant_equal(w1, got, O.quantize(w1), "refresh")
    # and equal to a fresh quantize of the same weight on the GPU
    fresh = quantize_gpu(w1)
    assert np.array_equal(fresh[0], got[0]) and np.array_equal(fresh[1], got[1])


def test_sentinels_and_guard_bytes():
    """Pre-filled outputs are fully overwritten; bytes around them are untouched."""
    n, k = 77, 336
    w = wl.random_weight_bits(n, k, sigma=0.3, seed=4)
    guard = 4096
    pbuf = torch.full((guard + n * k // 2 + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((guard + n * k // 16 + guard,), 0x7F, dtype=torch.uint8, device=DEV)  # e4m3 NaN
    gbuf = torch.full((64 + 1 + 63,), float("nan"), dtype=torch.float32, device=DEV)
    p = pbuf[guard:guard + n * k // 2].view(n, k // 2)
    s = sbuf[guard:guard + n * k // 16].view(n, k // 16)
    g = gbuf[64]
    B.nvfp4_refresh_inplace(dev_bf16(w), p, s, g)
    torch.cuda.synchronize()
    assert_quant_equal(w, (p.cpu().numpy(), s.cpu().numpy(), np.float32(g.item())), O.quantize(w), "sentinel")
    pb = pbuf.cpu().numpy()
    sb = sbuf.cpu().numpy()
    gb = gbuf.cpu().numpy()
    assert np.all(pb[:guard] == 0xA5) and np.all(pb[guard + n * k // 2:] == 0xA5)
    assert np.all(sb[:guard] == 0x7F) and np.all(sb[guard + n * k // 16:] == 0x7F)
    assert np.all(np.isnan(gb[:64])) and np.all(np.isnan(gb[65:]))


def test_deterministic():
    w = wl.random_weight_bits(512, 1024, sigma=0.02, seed=9)
    a = quantize_gpu(w)
    b = quantize_gpu(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and f32_bits(a[2]) == f32_bits(b[2])


def test_refresh_in_captured_graph_replays():
    """The refresh sequence has no memset node: capture it and replay with new weights."""
    n, k = 200, 512
    wbuf = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    p = torch.empty((n, k // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((n, k // 16), dtype=torch.float8_e4m3fn, device=DEV)
    g = torch.empty((), dtype=torch.float32, device=DEV)
    w0 = wl.random_weight_bits(n, k, sigma=0.02, seed=20)
    wbuf.copy_(dev_bf16(w0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.nvfp4_refresh_inplace(wbuf, p, s, g)    # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_refresh_inplace(wbuf, p, s, g)
    for seed in (21, 22, 23):
        wi = wl.random_weight_bits(n, k, sigma=0.02 * (seed - 19), seed=seed)
        wbuf.copy_(dev_bf16(wi))
        graph.replay()
        torch.cuda.synchronize()
        got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
        assert_quant_equal(wi, got, O.quantize(wi), f"graph replay {seed}")
        # eager work between replays
        eager = quantize_gpu(wi)
        assert np.array_equal(eager[0], got[0])


def test_scales_dtype_is_e4m3fn_and_layout():
    w = wl.random_weight_bits(10, 64, sigma=0.02, seed=2)
    p, s, g = B.nvfp4_quantize(dev_bf16(w))
    assert p.shape == (10, 32) and p.dtype == torch.uint8
    assert s.shape == (10, 4) and s.dtype == torch.float8_e4m3fn
    assert g.shape == () and g.dtype == torch.float32
    # torch's own decode of the scale bytes agrees with the oracle's E4M3 values
    want = O.e4m3_value(s.view(torch.uint8).cpu().numpy())
    assert np.array_equal(s.float().cpu().numpy().astype(np.float64), want)


def test_shape_error_is_valueerror():
    with pytest.raises(ValueError):
        B.nvfp4_quantize(torch.zeros((4, 24), dtype=torch.bfloat16, device=DEV))
