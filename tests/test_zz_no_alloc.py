"""GPU test of nvfp4_w4a4_gemm_noalloc, the W4A4 GEMM whose workspace is the
library's static device scratch (for callers that cannot allocate).

Through the C ABI (ctypes binding): its logits must equal those of
nvfp4_w4a4_gemm with a caller workspace bit for bit (same kernels, same
inputs), and lie within the W4A4 oracle's bound (vLLM modelopt.py,
KNvfp4Dynamic: NVFP4 activations with a static global input scale; alpha =
input_global_scale * weight_global_scale).  Two calls in a row share the
scratch, the second with a smaller input, so stale contents of the first call
must not leak into the second; a prefill-sized call and an oversized request
follow.
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, check_w4a4, dev_u8, host_bits

pytestmark = pytest.mark.gpu


def f32_dev(v):
    return torch.tensor(np.float32(v), dtype=torch.float32, device=DEV)


def case(m, n, k, seed):
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=seed)
    x = wl.random_activation_bits(m, k, seed=seed + 1)
    wp, ws, gw = O.quantize(w)
    gi = A.collapse_input_scale(np.float32([O.global_scale(O.weight_amax(x)) * np.float32(1.25)]))[0]
    xp, xs = A.quantize_activations(x, gi)
    bias = wl.bias_bits(n, seed=seed + 2, sigma=0.5) if seed % 2 else None
    return xp, xs, gi, wp, ws, gw, bias


def run_both(xp, xs, gi, wp, ws, gw, bias):
    m, n = xp.shape[0], wp.shape[0]
    dev = (dev_u8(xp), dev_u8(xs), f32_dev(gi), dev_u8(wp), dev_u8(ws), f32_dev(gw))
    b = None if bias is None else torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).to(DEV)
    ref = B.nvfp4_w4a4_gemm(*dev, bias=b)
    out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.nvfp4_w4a4_gemm_noalloc(*dev, out=out, bias=b)
    torch.cuda.synchronize()
    return host_bits(out), host_bits(ref)


def test_noalloc_matches_workspace_call_twice_in_a_row_then_smaller():
    for m, n, k, seed in [(48, 3000, 4096, 51), (5, 700, 1024, 52)]:
        xp, xs, gi, wp, ws, gw, bias = case(m, n, k, seed)
        got, ref = run_both(xp, xs, gi, wp, ws, gw, bias)
        assert np.array_equal(got, ref), f"noalloc differs from the workspace call at M={m} N={n} K={k}"
        check_w4a4(got, xp, xs, wp, ws, A.alpha(gi, gw), bias, label=f"noalloc M={m} N={n} K={k}")


def test_noalloc_prefill_size_and_largest_fitting_workspace():
    for m, n, k, seed in [(300, 515, 2048, 53), (255, 300, 8192, 54)]:
        assert 2 * m * k + 16 <= B.W4A4_SCRATCH_BYTES
        xp, xs, gi, wp, ws, gw, bias = case(m, n, k, seed)
        got, ref = run_both(xp, xs, gi, wp, ws, gw, bias)
        assert np.array_equal(got, ref), f"noalloc differs from the workspace call at M={m} N={n} K={k}"
        check_w4a4(got, xp, xs, wp, ws, A.alpha(gi, gw), bias, label=f"noalloc M={m} N={n} K={k}")


def test_noalloc_rejects_a_workspace_larger_than_the_scratch():
    m, n, k = 2048, 64, 1024
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    xp = torch.zeros((m, k // 2), dtype=torch.uint8, device=DEV)
    xs = torch.zeros((m, k // 16), dtype=torch.uint8, device=DEV)
    wp = torch.zeros((n, k // 2), dtype=torch.uint8, device=DEV)
    ws = torch.zeros((n, k // 16), dtype=torch.uint8, device=DEV)
    g = f32_dev(1.0)
    with pytest.raises(B.NVFP4Error, match="NVFP4_ERR_SCRATCH"):
        B.nvfp4_w4a4_gemm_noalloc(xp, xs, g, wp, ws, g, out=out)
