"""GPU parity at the full workload sizes, through the same entry points and
launch configurations bench.py times.

Quantization: every byte of packed codes and scales and the global scale's bits
against the oracle (quantized on a thread pool, same arithmetic).
GEMM: every logit of each decode M against the fp64 oracle; for the prefill
sizes (M = 4096, 8192), a sample of activation rows against all N and all rows
against a sample of vocabulary columns.  The same for NVFP4 W4A4 (activations
quantized with a static global input scale) at every decode M and the Qwen
prefill, and for the FP8 copy at the Qwen prefill.  One test per workload, so
each weight is generated and quantized once; each step prints its case first.
"""

import numpy as np
import pytest
import torch

import oracle.fp8_oracle as F
import oracle.nvfp4_oracle as O
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import (DEV, assert_quant_equal, check_fp8_gemm, check_gemm, check_w4a4, dev_bf16, dev_u8,
                      host_bits, oracle_quantize_threaded)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def say(msg):
    print(msg, flush=True)


def quantize_both(w, wb):
    wd = dev_bf16(wb)
    p, s, g = B.nvfp4_quantize(wd)
    torch.cuda.synchronize()
    gs = O.global_scale(O.weight_amax(wb))
    op, os_ = oracle_quantize_threaded(wb, gs)
    got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
    assert_quant_equal(wb, got, (op, os_, gs), w.name)
    return wd, (p, s, g), (op, os_, gs), got


def input_scale(xb):
    """A static global input scale for the activations: their amax/2688, as a
    checkpoint's calibrated input_scale would hold."""
    return O.global_scale(O.weight_amax(xb))


def decode_checks(w, xb, q, oq, ms):
    gi = input_scale(xb)
    gi_dev = torch.tensor(gi, device=DEV)
    for m in ms:
        say(f"[{w.name}] decode GEMM M={m}")
        x = xb[:m]
        y = host_bits(B.nvfp4_w4a16_gemm(dev_bf16(x), *q))
        check_gemm(y, x, *oq, label=f"{w.name} M={m}", argmax_min=0.999)
        say(f"[{w.name}] W4A4 GEMM M={m}")
        xp, xs = A.quantize_activations(x, gi)
        y4 = host_bits(B.nvfp4_w4a4_gemm(dev_u8(xp), dev_u8(xs), gi_dev, *q))
        check_w4a4(y4, xp, xs, oq[0], oq[1], A.alpha(gi, oq[2]), label=f"{w.name} W4A4 M={m}")


def prefill_checks(w, xb, q, oq, m):
    say(f"[{w.name}] prefill GEMM M={m}")
    y_dev = B.nvfp4_w4a16_gemm(dev_bf16(xb[:m]), *q)
    torch.cuda.synchronize()
    op, os_, gs = oq
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 126, replace=False)]))
    y_rows = host_bits(y_dev[torch.from_numpy(rows).to(DEV)])
    check_gemm(y_rows, xb[rows], op, os_, gs, label=f"{w.name} rows", argmax_min=0.999)
    cols = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, 254, replace=False)]))
    y_cols = host_bits(y_dev[:, torch.from_numpy(cols).to(DEV)])
    check_gemm(y_cols, xb[:m], op[cols], os_[cols], gs, label=f"{w.name} cols", argmax_min=0.0)
    del y_dev


def test_llama3_8b():
    w = wl.WORKLOADS["llama3_8b"]
    say(f"[{w.name}] generating {w.n}x{w.k}")
    wb, xb = wl.weight_bits(w), wl.activation_bits(w)
    say(f"[{w.name}] quantize parity")
    _, q, oq, _ = quantize_both(w, wb)
    decode_checks(w, xb, q, oq, w.ms)


def test_llama3_70b_with_refresh_and_graph():
    """70B shape: decode parity, then W' = W + N(0, 1e-3), an in-place refresh,
    and a GEMM graph captured before the refresh that computes the new logits."""
    w = wl.WORKLOADS["llama3_70b"]
    say(f"[{w.name}] generating {w.n}x{w.k}")
    wb, xb = wl.weight_bits(w), wl.activation_bits(w)
    say(f"[{w.name}] quantize parity")
    wd, q, oq, _ = quantize_both(w, wb)
    decode_checks(w, xb, q, oq, w.ms)
    say(f"[{w.name}] refresh in place + graph replay")
    p, s, g = q
    ptrs = (p.data_ptr(), s.data_ptr(), g.data_ptr())
    x = xb[:1]
    xd = dev_bf16(x)
    out = torch.empty((1, w.n), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.nvfp4_w4a16_gemm(xd, p, s, g, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_w4a16_gemm(xd, p, s, g, out=out)
    w2 = wl.refresh_weight_bits(w, wb)
    wd.copy_(dev_bf16(w2))
    B.nvfp4_refresh_inplace(wd, p, s, g)
    graph.replay()
    torch.cuda.synchronize()
    assert (p.data_ptr(), s.data_ptr(), g.data_ptr()) == ptrs
    gs2 = O.global_scale(O.weight_amax(w2))
    op2, os2 = oracle_quantize_threaded(w2, gs2)
    got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
    assert_quant_equal(w2, got, (op2, os2, gs2), "70b refresh")
    check_gemm(host_bits(out), x, op2, os2, gs2, label="70b graph after refresh")


def sample_rows_cols(m, n, seed=7):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 126, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 254, replace=False)]))
    return rows, cols


def test_qwen_prefill():
    w = wl.WORKLOADS["qwen_prefill"]
    say(f"[{w.name}] generating {w.n}x{w.k}")
    wb, xb = wl.weight_bits(w), wl.activation_bits(w)
    say(f"[{w.name}] quantize parity")
    wd, q, oq, _ = quantize_both(w, wb)
    prefill_checks(w, xb, q, oq, 4096)
    m = 4096
    rows, cols = sample_rows_cols(m, w.n)
    rt, ct = torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)

    say(f"[{w.name}] W4A4 prefill M={m}")
    gi = input_scale(xb[:m])
    xp, xs = A.quantize_activations(xb[:m], gi)
    y4 = B.nvfp4_w4a4_gemm(dev_u8(xp), dev_u8(xs), torch.tensor(gi, device=DEV), *q)
    torch.cuda.synchronize()
    a = A.alpha(gi, oq[2])
    check_w4a4(host_bits(y4[rt]), xp[rows], xs[rows], oq[0], oq[1], a, label="qwen W4A4 rows")
    check_w4a4(host_bits(y4[:, ct]), xp, xs, oq[0][cols], oq[1][cols], a, label="qwen W4A4 cols", argmax_min=0.0)
    del y4

    say(f"[{w.name}] FP8 copy: weight quantization parity + prefill M={m}")
    qw, sw = B.nvfp4_fp8_quantize_rows(wd)
    torch.cuda.synchronize()
    owq, ows = F.quantize_rows(wb)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), ows.view(np.uint32))
    assert np.array_equal(qw.view(torch.uint8).cpu().numpy(), owq)
    xq, xsc = F.quantize_rows(xb[:m])
    y8 = B.nvfp4_fp8_gemm(dev_u8(xq), torch.from_numpy(xsc).to(DEV), dev_u8(owq), torch.from_numpy(ows).to(DEV))
    torch.cuda.synchronize()
    check_fp8_gemm(host_bits(y8[rt]), xq[rows], xsc[rows], owq, ows, label="qwen FP8 rows")
    check_fp8_gemm(host_bits(y8[:, ct]), xq, xsc, owq[cols], ows[cols], label="qwen FP8 cols", argmax_min=0.0)


def test_heavy_tail():
    w = wl.WORKLOADS["heavy_tail"]
    say(f"[{w.name}] generating {w.n}x{w.k}")
    wb, xb = wl.weight_bits(w), wl.activation_bits(w)
    say(f"[{w.name}] quantize parity")
    _, q, oq, got = quantize_both(w, wb)
    # zero row -> zero codes and scales; grid row keeps the generator's codes
    assert not got[0][0].any() and not got[1][0].any()
    g_row = wl.bf16_bits_to_f32(wl.grid_row_bits(w.k)).astype(np.float64)
    mag = O.e2m1_magnitude_code(np.abs(g_row).astype(np.float32))
    want = np.where((g_row < 0) & (mag != 0), mag | 8, mag).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(got[0][-1:])[0], want)
    decode_checks(w, xb, q, oq, (1,))
    prefill_checks(w, xb, q, oq, 8192)
