"""GPU parity: nvfp4_w4a16_gemm against the fp64 dequantize-then-matmul oracle.

Tolerance (per element): |y - y64| <= 1e-3 * ||x_m||_2 * ||w_deq_n||_2, plus a
tight bound for fp32 accumulation of exact products and one bf16 rounding;
tie-aware per-row argmax agreement.  Closed forms (one-hot rows, zero rows)
are bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, check_gemm, dev_bf16, gemm_gpu, host_bits, oracle_quantize_threaded, upload_quant

pytestmark = pytest.mark.gpu


def setup(n, k, sigma=0.02, seed=0):
    w = wl.random_weight_bits(n, k, sigma=sigma, seed=seed)
    packed, scales, gs = O.quantize(w)
    return w, packed, scales, gs, upload_quant(packed, scales, gs)


def test_tiny_workload_end_to_end():
    """Quantize on the GPU, then GEMM on the GPU's own buffers."""
    w = wl.WORKLOADS["tiny"]
    wb = wl.weight_bits(w)
    x = wl.activation_bits(w)
    p, s, g = B.nvfp4_quantize(dev_bf16(wb))
    y = host_bits(B.nvfp4_w4a16_gemm(dev_bf16(x), p, s, g))
    packed, scales, gs = O.quantize(wb)
    check_gemm(y, x, packed, scales, gs, label="tiny", argmax_min=1.0)


# decode (M <= 64) and prefill (M > 64) paths, ragged M, N and K; K % 128 == 64 and
# K = 128 (a single weight superblock) exercise both prefill kernels
@pytest.mark.parametrize("m", [1, 2, 4, 15, 16, 17, 33, 48, 64, 65, 100, 128, 129, 300])
@pytest.mark.parametrize("n,k", [(1024, 512), (1027, 272), (77, 4096), (200, 48), (5, 16),
                                 (300, 7168), (64, 8448), (515, 320), (300, 128), (260, 64), (100, 192)])
def test_shapes(m, n, k):
    w, packed, scales, gs, q = setup(n, k, seed=m)
    x = wl.random_activation_bits(m, k, seed=n)
    y = gemm_gpu(x, q)
    check_gemm(y, x, packed, scales, gs, label=f"m={m} n={n} k={k}", argmax_min=0.99 if n < 20 else 0.999)


# M <= 16 with x too large for LDS (and M <= 2 past the dot kernel's K): the
# panel kernel, or the phased x-resident kernel where a phase of x fits (M =
# 5 at K = 16384: two phases; M = 16 at K = 16384: eight), several 512-row
# blocks with a ragged last one, K of 20 and 32 K columns, bias on one row
# count
@pytest.mark.parametrize("m", [1, 2, 5, 12, 16])
@pytest.mark.parametrize("n,k", [(1100, 16384), (700, 10240)])
def test_decode_panel_rows_up_to_16(m, n, k):
    w, packed, scales, gs, q = setup(n, k, seed=m + 7)
    x = wl.random_activation_bits(m, k, seed=n + m)
    bias = wl.bias_bits(n, seed=m, sigma=0.5) if m == 12 else None
    y = gemm_gpu(x, q, bias)
    check_gemm(y, x, packed, scales, gs, bias_bits=bias, label=f"panel m={m} n={n} k={k}")


# 3 <= M <= 16 with x too large for LDS whole but K a multiple of 2048: the
# phased x-resident kernel (x held one column range at a time, 16
# wavefronts).  Two phases at K = 4096, four at K = 8192; up to 2 tiles per
# wavefront at N = 70000, up to 4 (3 used) at N = 131100, one at N = 40000,
# wavefronts without tiles at N = 3001; bias
@pytest.mark.parametrize("m,n,k,with_bias", [(15, 131100, 4096, False), (16, 70000, 4096, True),
                                             (16, 40000, 8192, True), (9, 3001, 8192, False),
                                             (16, 3001, 4096, True)])
def test_decode_x_in_phases(m, n, k, with_bias):
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=m + 3)
    gs = O.global_scale(O.weight_amax(w))
    packed, scales = oracle_quantize_threaded(w, gs)
    q = upload_quant(packed, scales, gs)
    x = wl.random_activation_bits(m, k, seed=n + 5)
    bias = wl.bias_bits(n, seed=m, sigma=0.5) if with_bias else None
    y = gemm_gpu(x, q, bias)
    check_gemm(y, x, packed, scales, gs, bias_bits=bias, label=f"phases m={m} n={n} k={k}")


# decode with more 512-row blocks than the GPU has compute units, so that
# workgroups walk several blocks (N = 140000 > 256 * 512), ragged last block
@pytest.mark.parametrize("m", [3, 24, 33, 64])
def test_decode_more_row_blocks_than_compute_units(m):
    n, k = 140000, 1024
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=m + 40)
    gs = O.global_scale(O.weight_amax(w))
    packed, scales = oracle_quantize_threaded(w, gs)
    q = upload_quant(packed, scales, gs)
    x = wl.random_activation_bits(m, k, seed=m + 41)
    y = gemm_gpu(x, q)
    check_gemm(y, x, packed, scales, gs, label=f"blocks m={m} n={n} k={k}")


# more 256 x 256 prefill tiles than the GPU has compute units (several waves
# of workgroups), every logit checked: 2 to 6 steps of 64 k per tile, ragged
# M and N, odd N, bias.  On a 256-CU GPU the last partial round of tiles is
# split 2 ways (1900 x 20000, 1100 x 30001), 4 ways (1000 x 35228) and 8 ways
# (800 x 33000) over narrower workgroups; 200 x 102400 runs unsplit.
@pytest.mark.parametrize("m,n,k,with_bias", [(1900, 20000, 192, False), (800, 33000, 256, False),
                                             (1100, 30001, 320, True), (1000, 35228, 384, True),
                                             (200, 102400, 128, False)])
def test_prefill_many_tiles(m, n, k, with_bias):
    w, packed, scales, gs, q = setup(n, k, seed=m)
    x = wl.random_activation_bits(m, k, seed=n)
    bias = wl.bias_bits(n, seed=k, sigma=0.5) if with_bias else None
    y = gemm_gpu(x, q, bias)
    check_gemm(y, x, packed, scales, gs, bias_bits=bias, label=f"tiles m={m} n={n} k={k}")


@pytest.mark.parametrize("m", [1, 8, 64, 200])
def test_bias(m):
    n, k = 515, 1024
    w, packed, scales, gs, q = setup(n, k, seed=3)
    x = wl.random_activation_bits(m, k, seed=4)
    bias = wl.bias_bits(n, seed=5, sigma=0.5)
    y = gemm_gpu(x, q, bias)
    check_gemm(y, x, packed, scales, gs, bias_bits=bias, label=f"bias m={m}")


@pytest.mark.parametrize("m", [1, 7, 64, 70, 256])
def test_onehot_rows_are_exact(m):
    """x = e_k gives y[m, n] = bf16(fl32(gs * (E2M1 * scale))) in any summation order."""
    n, k = 333, 512
    w, packed, scales, gs, q = setup(n, k, sigma=0.1, seed=6)
    ks = np.random.default_rng(m).integers(0, k, size=m)
    x = np.zeros((m, k), np.uint16)
    x[np.arange(m), ks] = 0x3F80      # 1.0
    y = wl.bf16_bits_to_f32(gemm_gpu(x, q)).astype(np.float64)
    codes = O.unpack_codes(packed)
    for i, kk in enumerate(ks):
        d = O.e2m1_value(codes[:, kk]) * O.e4m3_value(scales[:, kk // 16])   # exact in fp32
        want = O.bf16_round_rne(np.float32(gs) * d.astype(np.float32))
        assert np.array_equal(y[i], want), f"row {i} k={kk}"


@pytest.mark.parametrize("m", [3, 90])
def test_zero_weight_rows_give_zero_or_bias(m):
    n, k = 64, 256
    w = wl.random_weight_bits(n, k, seed=7)
    w[[0, 17, 63]] = 0
    packed, scales, gs = O.quantize(w)
    q = upload_quant(packed, scales, gs)
    x = wl.random_activation_bits(m, k, seed=8)
    y = wl.bf16_bits_to_f32(gemm_gpu(x, q)).astype(np.float64)
    assert np.all(y[:, [0, 17, 63]] == 0)
    bias = wl.bias_bits(n, seed=9)
    yb = gemm_gpu(x, q, bias)
    assert np.array_equal(yb[:, [0, 17, 63]], np.broadcast_to(bias[[0, 17, 63]], (m, 3)))


def test_m_zero_is_empty():
    n, k = 64, 256
    _, _, _, _, q = setup(n, k)
    y = B.nvfp4_w4a16_gemm(torch.empty((0, k), dtype=torch.bfloat16, device=DEV), *q)
    assert y.shape == (0, n)


@pytest.mark.parametrize("m", [5, 64, 130])
def test_deterministic_and_guarded_output(m):
    n, k = 1031, 1024
    _, packed, scales, gs, q = setup(n, k, seed=10)
    x = dev_bf16(wl.random_activation_bits(m, k, seed=11))
    guard = 2048
    buf = torch.full((guard + m * n + guard,), 0x7FC1, dtype=torch.int16, device=DEV)   # a NaN pattern
    out = buf[guard:guard + m * n].view(torch.bfloat16).view(m, n)
    B.nvfp4_w4a16_gemm(x, *q, out=out)
    y1 = host_bits(out)
    B.nvfp4_w4a16_gemm(x, *q, out=out)
    y2 = host_bits(out)
    assert np.array_equal(y1, y2)
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 0x7FC1) and np.all(b[guard + m * n:] == 0x7FC1)
    check_gemm(y1, wl.random_activation_bits(m, k, seed=11), packed, scales, gs, label="guarded")


def test_graph_replay_sees_refreshed_weights():
    """A graph that captured the GEMM keeps working after an in-place refresh."""
    n, k, m = 1024, 512, 8
    w0 = wl.random_weight_bits(n, k, sigma=0.02, seed=30)
    w1 = wl.random_weight_bits(n, k, sigma=0.03, seed=31)
    x = wl.random_activation_bits(m, k, seed=32)
    p, s, g = B.nvfp4_quantize(dev_bf16(w0))
    xd = dev_bf16(x)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.nvfp4_w4a16_gemm(xd, p, s, g, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_w4a16_gemm(xd, p, s, g, out=out)
    for wi in (w0, w1, w0):
        B.nvfp4_refresh_inplace(dev_bf16(wi), p, s, g)
        graph.replay()
        torch.cuda.synchronize()
        packed, scales, gs = O.quantize(wi)
        check_gemm(host_bits(out), x, packed, scales, gs, label="graph replay")


def test_gpu_quantized_buffers_match_oracle_buffers_in_gemm():
    """Running the GEMM on GPU-quantized and on oracle-quantized buffers gives equal bytes."""
    n, k, m = 2048, 1024, 33
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=40)
    x = wl.random_activation_bits(m, k, seed=41)
    packed, scales, gs = O.quantize(w)
    y_oracle_buf = gemm_gpu(x, upload_quant(packed, scales, gs))
    p, s, g = B.nvfp4_quantize(dev_bf16(w))
    y_gpu_buf = gemm_gpu(x, (p, s, g))
    assert np.array_equal(y_oracle_buf, y_gpu_buf)


@pytest.mark.parametrize("m,k", [(8, 1024), (40, 1024), (16, 8192)])
def test_decode_activation_rows_of_extreme_magnitude(m, k):
    """Decode rows whose magnitudes span the bf16 range: zeros, ~2^100, ~2^-100,
    a mix of 2^20 and 2^-20 within one row, one huge element among tiny ones,
    and rows whose largest elements come only in the last (or only in the
    first) columns.  M = 8 keeps x resident in LDS (f16 products with a
    per-row exponent); M = 16 at K = 8192 holds it in four 2048-column
    phases with the exponent taken from the whole row; M = 40 (two
    512-column panels) takes the panel kernel."""
    n = 1027
    _, packed, scales, gs, q = setup(n, k, seed=12)
    rng = np.random.default_rng(13)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    xf[0] = 0.0
    xf[1] *= np.float32(2.0 ** 100)
    xf[2] *= np.float32(2.0 ** -100)
    xf[3] *= np.where(rng.random(k) < 0.5, np.float32(2.0 ** 20), np.float32(2.0 ** -20))
    xf[4] *= np.float32(2.0 ** -60)
    xf[4, 17] = np.float32(3.0e4)
    xf[5, : k - 64] *= np.float32(2.0 ** -40)
    xf[5, k - 64:] *= np.float32(2.0 ** 40)
    xf[6, :64] *= np.float32(2.0 ** 40)
    xf[6, 64:] *= np.float32(2.0 ** -40)
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = gemm_gpu(x, q)
    assert not np.any(y[0] & 0x7FFF), "zero row must give zero logits"
    check_gemm(y, x, packed, scales, gs, label="extreme rows", argmax_min=0.0)
