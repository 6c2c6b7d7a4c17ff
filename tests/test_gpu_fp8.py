"""GPU parity of the FP8 lm_head copy against oracle/fp8_oracle.py.

Row quantization (weights per output row, activations per token): every byte
and every scale bit.  GEMM: every logit against the float64 reference of the
same quantized operands, within the norm bound and a tight bound set by
the fp8 MFMA's accumulation precision (see check_fp8_gemm), and the argmax.
"""

import numpy as np
import pytest
import torch

import oracle.fp8_oracle as F
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, check_fp8_gemm, dev_bf16, dev_u8, f32_bits, host_bits

pytestmark = pytest.mark.gpu


def quant_gpu(bits):
    q, s = B.nvfp4_fp8_quantize_rows(dev_bf16(bits))
    torch.cuda.synchronize()
    return q.view(torch.uint8).cpu().numpy(), s.cpu().numpy()


def assert_quant_equal(bits, label):
    q, s = quant_gpu(bits)
    oq, os_ = F.quantize_rows(bits)
    bad_s = np.flatnonzero(s.view(np.uint32) != os_.view(np.uint32))
    assert bad_s.size == 0, f"{label}: {bad_s.size} scales differ, first row {bad_s[0]}: {s[bad_s[0]]!r} vs {os_[bad_s[0]]!r}"
    bad = np.argwhere(q != oq)
    if bad.size:
        i, j = bad[0]
        v = wl.bf16_bits_to_f32(bits[i, j:j + 1])[0]
        raise AssertionError(f"{label}: {len(bad)} bytes differ; first [{i},{j}] x={v!r} scale={os_[i]!r} "
                             f"gpu={q[i, j]:#04x} oracle={oq[i, j]:#04x}")
    return oq, os_                                     # equal to the GPU's; references use the oracle's


@pytest.mark.parametrize("r,k", [(1, 16), (37, 96), (1027, 1024), (7, 3072), (300, 4112), (5, 8192), (3, 8208)])
def test_quantize_rows_bit_exact(r, k):
    bits = wl.random_weight_bits(r, k, sigma=0.05, seed=r + k)
    assert_quant_equal(bits, f"{r}x{k}")


def test_quantize_rows_special_rows():
    k = 64
    rng = np.random.default_rng(8)
    rows = []
    rows.append(np.zeros(k, np.float32))                                  # zero row
    v = np.zeros(k, np.float32); v[3] = -0.0; v[5] = 1.0; rows.append(v)  # -0 and one value
    v = rng.standard_normal(k).astype(np.float32) * 1e-3; v[0] = 3.0e4; rows.append(v)   # subnormal codes
    v = rng.standard_normal(k).astype(np.float32) * 2.0 ** 100; rows.append(v)
    v = rng.standard_normal(k).astype(np.float32) * 2.0 ** -100; rows.append(v)
    v = np.full(k, -7.0, np.float32); rows.append(v)
    # values landing exactly between two codes after scaling by 448 / 448
    codes = np.arange(0x08, 0x7E, dtype=np.uint8)
    mids = ((F.e4m3_decode_signed(codes[:-1]) + F.e4m3_decode_signed(codes[1:])) / 2)[:k - 1]
    v = np.concatenate([[448.0], mids]).astype(np.float32); rows.append(v)
    bits = torch.from_numpy(np.stack(rows)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = assert_quant_equal(bits, "special rows")
    assert not q[0].any()
    assert q[1, 3] == 0x80 and q[1, 5] == 0x7E


@pytest.mark.parametrize("m", [1, 2, 4, 17, 32, 64, 65, 130, 300])
@pytest.mark.parametrize("n,k", [(1027, 512), (128, 48), (300, 1040), (2053, 4096)])
def test_gemm_matches_oracle(m, n, k):
    """M = 1 (K <= 4096) and M = 2 (K <= 2048) run the VALU dot kernel
    (segments past K in the last 64-lane round: K = 48, 1040), the rest the
    MFMA kernels."""
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=n + k)
    x = wl.random_activation_bits(m, k, seed=m + 7)
    wq, ws = F.quantize_rows(w)
    xq, xs = F.quantize_rows(x)
    y = B.nvfp4_fp8_gemm(dev_u8(xq), torch.from_numpy(xs).to(DEV), dev_u8(wq), torch.from_numpy(ws).to(DEV))
    check_fp8_gemm(host_bits(y), xq, xs, wq, ws, label=f"M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,k,with_bias", [(1, 3000, 8192, True), (2, 2100, 8192, False),
                                             (5, 3000, 2560, True), (3, 1100, 7168, False), (20, 2100, 1536, True),
                                             (4, 1027, 512, False),
                                             (3, 140000, 512, True), (20, 70000, 512, False), (28, 140000, 512, True),
                                             (16, 1300, 8192, False), (24, 1030, 8192, True), (40, 2100, 1024, False),
                                             (40, 70000, 512, True), (64, 900, 8192, True)])
def test_ring_kernel_panels_blocks_and_bias(m, n, k, with_bias):
    """M <= 64 with K % 512 == 0 runs the register-ring kernel (at M = 1, 2
    beyond the dot kernel's K): several x panels per block at K = 8192 (4 at
    M <= 16, 8 at M <= 32, 16 beyond),
    more 512-row (M <= 32) or 256-row (M > 32) blocks than compute units at
    N = 140000 / 70000, rows past N and M in the last tiles, and the bias;
    K not a multiple of the panel width (a partial last panel: K = 2560 and
    7168 at M <= 16, 1536 at M <= 32) and K below it (K = 512 at M <= 16)."""
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=n + 3 * k)
    x = wl.random_activation_bits(m, k, seed=m + 11)
    wq, ws = F.quantize_rows(w)
    xq, xs = F.quantize_rows(x)
    bias = wl.random_weight_bits(1, n, sigma=0.5, seed=5)[0] if with_bias else None
    y = B.nvfp4_fp8_gemm(dev_u8(xq), torch.from_numpy(xs).to(DEV), dev_u8(wq), torch.from_numpy(ws).to(DEV),
                         bias=dev_bf16(bias) if with_bias else None)
    check_fp8_gemm(host_bits(y), xq, xs, wq, ws, bias_bits=bias, label=f"ring M={m} N={n} K={k}")


def test_gemm_with_bias_end_to_end():
    """GPU quantization of both operands, then the GEMM with a bias."""
    n, k, m = 515, 320, 9
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=1)
    x = wl.random_activation_bits(m, k, seed=2)
    bias = wl.random_weight_bits(1, n, sigma=0.5, seed=3)[0]
    wq, ws = assert_quant_equal(w, "w")
    xq, xs = assert_quant_equal(x, "x")
    qw, sw = B.nvfp4_fp8_quantize_rows(dev_bf16(w))
    qx, sx = B.nvfp4_fp8_quantize_rows(dev_bf16(x))
    y = B.nvfp4_fp8_gemm(qx, sx, qw, sw, bias=dev_bf16(bias))
    check_fp8_gemm(host_bits(y), xq, xs, wq, ws, bias, label="bias")


@pytest.mark.parametrize("m,n,k", [(65, 300, 64), (300, 515, 192), (257, 1027, 320), (513, 260, 128), (300, 100, 256)])
def test_prefill_tiles_odd_step_counts_with_bias(m, n, k):
    """M > 64 with K % 64 == 0 (the 256 x 256 tile kernel): 1, 2, 3, 4 and 5
    64-byte k steps (odd counts end on the loop's tail step), ragged M and N,
    N below one tile, several M tiles, and a bias."""
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=n * 3 + k)
    x = wl.random_activation_bits(m, k, seed=m * 5 + k)
    bias = wl.random_weight_bits(1, n, sigma=0.5, seed=n + 1)[0]
    wq, ws = F.quantize_rows(w)
    xq, xs = F.quantize_rows(x)
    y = B.nvfp4_fp8_gemm(dev_u8(xq), torch.from_numpy(xs).to(DEV), dev_u8(wq), torch.from_numpy(ws).to(DEV),
                         bias=dev_bf16(bias))
    check_fp8_gemm(host_bits(y), xq, xs, wq, ws, bias, label=f"prefill M={m} N={n} K={k}")


def test_gemm_empty_batch_and_scale_bits():
    w = wl.random_weight_bits(64, 32, seed=5)
    qw, sw = B.nvfp4_fp8_quantize_rows(dev_bf16(w))
    y = B.nvfp4_fp8_gemm(torch.empty((0, 32), dtype=torch.uint8, device=DEV),
                         torch.empty((0,), dtype=torch.float32, device=DEV), qw, sw)
    assert y.shape == (0, 64)
    _, os_ = F.quantize_rows(w)
    assert all(f32_bits(a) == f32_bits(b) for a, b in zip(sw.cpu().numpy(), os_))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_size_8b_shape():
    """128256 x 4096 weight: every byte and scale; every logit at M = 1, 8, 32, 64."""
    w = wl.WORKLOADS["llama3_8b"]
    wb = wl.weight_bits(w)
    xb = wl.activation_bits(w)
    q, s = quant_gpu(wb)
    oq, os_ = F.quantize_rows(wb)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q, oq)
    wdev, sdev = dev_u8(oq), torch.from_numpy(os_).to(DEV)
    for m in w.ms:                                     # 1, 8, 32, 64, as the bench times them
        xq, xs = F.quantize_rows(xb[:m])
        y = B.nvfp4_fp8_gemm(dev_u8(xq), torch.from_numpy(xs).to(DEV), wdev, sdev)
        check_fp8_gemm(host_bits(y), xq, xs, oq, os_, label=f"8B M={m}")
