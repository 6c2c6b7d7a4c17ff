"""GPU parity of NVFP4 W4A4 against oracle/nvfp4_w4a4_oracle.py.

Activation quantization with a given global scale: every packed byte and
scale byte.  GEMM: every logit against the float64 reference of the same
NVFP4 operands within the float32-accumulation bound (products of two exact
bf16 values are exact in float32) plus one bf16 rounding; alpha's bits.
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, check_w4a4, dev_bf16, dev_u8, f32_bits, host_bits

pytestmark = pytest.mark.gpu


def f32_dev(v):
    return torch.tensor(np.float32(v), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("m,k", [(1, 16), (4, 512), (64, 4096), (130, 1040), (3, 8192)])
@pytest.mark.parametrize("gs_in", ["own", 2.0 ** -8, 3.7e-4])
def test_activation_quantization_bit_exact(m, k, gs_in):
    x = wl.random_activation_bits(m, k, seed=m * 7 + k)
    g = O.global_scale(O.weight_amax(x)) if gs_in == "own" else np.float32(gs_in)
    p, s = B.nvfp4_quantize_activations(dev_bf16(x), f32_dev(g))
    torch.cuda.synchronize()
    op, os_ = A.quantize_activations(x, g)
    assert np.array_equal(s.view(torch.uint8).cpu().numpy(), os_)
    assert np.array_equal(p.cpu().numpy(), op)


@pytest.mark.parametrize("m", [1, 2, 8, 40, 64, 65, 300])
@pytest.mark.parametrize("n,k", [(1027, 512), (300, 1040), (515, 320)])
def test_w4a4_gemm_matches_oracle(m, n, k):
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=n + k)
    x = wl.random_activation_bits(m, k, seed=m + 3)
    wp, ws, gw = O.quantize(w)
    gi = A.collapse_input_scale(np.float32([O.global_scale(O.weight_amax(x)) * np.float32(1.25)]))[0]
    xp, xs = A.quantize_activations(x, gi)
    y = B.nvfp4_w4a4_gemm(dev_u8(xp), dev_u8(xs), f32_dev(gi), dev_u8(wp), dev_u8(ws), f32_dev(gw))
    check_w4a4(host_bits(y), xp, xs, wp, ws, A.alpha(gi, gw), label=f"M={m} N={n} K={k}")


def test_w4a4_end_to_end_with_bias_and_workspace_reuse():
    n, k = 1027, 1024
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=11)
    bias = wl.random_weight_bits(1, n, sigma=0.5, seed=12)[0]
    pw, sw, gw = B.nvfp4_quantize(dev_bf16(w))
    owp, ows, ogw = O.quantize(w)                      # the reference uses the oracle's quantization
    assert np.array_equal(pw.cpu().numpy(), owp) and np.array_equal(sw.view(torch.uint8).cpu().numpy(), ows)
    assert f32_bits(gw.item()) == f32_bits(ogw)
    ws_buf = torch.empty((B.load_library().nvfp4_w4a4_workspace_bytes(64, k),), dtype=torch.uint8, device=DEV)
    gi = np.float32(2.0 ** -7)
    for m in (64, 5):                                  # the second call reuses a larger workspace
        x = wl.random_activation_bits(m, k, seed=20 + m)
        xp, xs = B.nvfp4_quantize_activations(dev_bf16(x), f32_dev(gi))
        y = B.nvfp4_w4a4_gemm(xp, xs, f32_dev(gi), pw, sw, gw, bias=dev_bf16(bias), workspace=ws_buf)
        torch.cuda.synchronize()
        a_dev = ws_buf[2 * m * k:2 * m * k + 4].view(torch.float32).item()
        assert f32_bits(a_dev) == f32_bits(A.alpha(gi, ogw))
        op, os_ = A.quantize_activations(x, gi)
        assert np.array_equal(xp.cpu().numpy(), op) and np.array_equal(xs.view(torch.uint8).cpu().numpy(), os_)
        check_w4a4(host_bits(y), op, os_, owp, ows, A.alpha(gi, ogw), bias, label=f"e2e M={m}")
