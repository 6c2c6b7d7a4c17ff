"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Quantization: every byte of packed codes and scales and the global scale's bits
against the oracle (quantized on a thread pool, same arithmetic).
GEMM: every logit of each decode M against the fp64 oracle; for prefill sizes
(M = 4096, 8192), a sample of activation rows against all N and all rows
against a sample of vocabulary columns.  Each test prints its case first.
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import (DEV, assert_quant_equal, check_gemm, dev_bf16, host_bits,
                      oracle_quantize_threaded)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

_cache = {}


def prepared(name):
    """Weight, activations, GPU quantization and oracle quantization of a workload."""
    if name in _cache:
        return _cache[name]
    _cache.clear()
    torch.cuda.empty_cache()
    w = wl.WORKLOADS[name]
    print(f"\n[{name}] generating {w.n}x{w.k}", flush=True)
    wb = wl.weight_bits(w)
    xb = wl.activation_bits(w)
    wd = dev_bf16(wb)
    p, s, g = B.nvfp4_quantize(wd)
    torch.cuda.synchronize()
    gs = O.global_scale(O.weight_amax(wb))
    op, os_ = oracle_quantize_threaded(wb, gs)
    _cache[name] = dict(w=w, wb=wb, xb=xb, wd=wd, q=(p, s, g), oracle=(op, os_, gs))
    return _cache[name]


@pytest.mark.parametrize("name", ["llama3_8b", "llama3_70b", "qwen_prefill", "heavy_tail"])
def test_quantize_full(name):
    d = prepared(name)
    print(f"[{name}] quantize parity", flush=True)
    p, s, g = d["q"]
    got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
    assert_quant_equal(d["wb"], got, d["oracle"], name)
    if name == "heavy_tail":
        # zero row -> zero codes and scales; grid row keeps the generator's codes
        assert not got[0][0].any() and not got[1][0].any()
        g_row = wl.bf16_bits_to_f32(wl.grid_row_bits(d["w"].k)).astype(np.float64)
        mag = O.e2m1_magnitude_code(np.abs(g_row).astype(np.float32))
        want = np.where((g_row < 0) & (mag != 0), mag | 8, mag).astype(np.uint8)
        assert np.array_equal(O.unpack_codes(got[0][-1:])[0], want)


DECODE = [("llama3_8b", m) for m in (1, 8, 32, 64)] + [("llama3_70b", m) for m in (1, 16, 64)] + \
         [("heavy_tail", 1)]


@pytest.mark.parametrize("name,m", DECODE)
def test_decode_gemm_full(name, m):
    d = prepared(name)
    print(f"[{name}] decode GEMM M={m}", flush=True)
    x = d["xb"][:m]
    y = host_bits(B.nvfp4_w4a16_gemm(dev_bf16(x), *d["q"]))
    op, os_, gs = d["oracle"]
    check_gemm(y, x, op, os_, gs, label=f"{name} M={m}", argmax_min=0.999)


@pytest.mark.parametrize("name", ["qwen_prefill", "heavy_tail"])
def test_prefill_gemm_sampled(name):
    d = prepared(name)
    w = d["w"]
    m = w.ms[0]
    print(f"[{name}] prefill GEMM M={m}", flush=True)
    y_dev = B.nvfp4_w4a16_gemm(dev_bf16(d["xb"]), *d["q"])
    torch.cuda.synchronize()
    op, os_, gs = d["oracle"]
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 254, replace=False)]))
    y_rows = host_bits(y_dev[torch.from_numpy(rows).to(DEV)])
    check_gemm(y_rows, d["xb"][rows], op, os_, gs, label=f"{name} rows", argmax_min=0.999)
    cols = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, 254, replace=False)]))
    y_cols = host_bits(y_dev[:, torch.from_numpy(cols).to(DEV)])
    check_gemm(y_cols, d["xb"], op[cols], os_[cols], gs, label=f"{name} cols", argmax_min=0.0)
    del y_dev


def test_refresh_70b_with_graph():
    """70B shape: W' = W + N(0, 1e-3); in-place refresh; a GEMM graph captured
    before the refresh computes the new logits on replay."""
    d = prepared("llama3_70b")
    w = d["w"]
    print("[llama3_70b] refresh in place", flush=True)
    p, s, g = d["q"]
    ptrs = (p.data_ptr(), s.data_ptr(), g.data_ptr())
    x = d["xb"][:1]
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
    w2 = wl.refresh_weight_bits(w, d["wb"])
    d["wd"].copy_(dev_bf16(w2))
    B.nvfp4_refresh_inplace(d["wd"], p, s, g)
    graph.replay()
    torch.cuda.synchronize()
    assert (p.data_ptr(), s.data_ptr(), g.data_ptr()) == ptrs
    gs2 = O.global_scale(O.weight_amax(w2))
    op2, os2 = oracle_quantize_threaded(w2, gs2)
    got = (p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.item()))
    assert_quant_equal(w2, got, (op2, os2, gs2), "70b refresh")
    check_gemm(host_bits(out), x, op2, os2, gs2, label="70b graph after refresh")
    _cache.clear()
