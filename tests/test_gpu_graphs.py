"""HIP-graph capture of the checkpoint, FP8, W4A4 and expert-layer calls: each sequence is
captured once, then replayed with new inputs written into the captured
buffers, with eager work between replays; every replay must equal the eager
result (and, for the quantizers, the oracle)."""

import numpy as np
import pytest
import torch

import oracle.fp8_oracle as F
import oracle.nvfp4_import_oracle as I
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, dev_bf16, dev_u8, f32_bits, host_bits

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                           # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def test_fp8_linear_graph_replays():
    n, k, m = 515, 320, 9
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=31)
    qw, sw = B.nvfp4_fp8_quantize_rows(dev_bf16(w))
    xbuf = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
    qx = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=DEV)
    sx = torch.empty((m,), dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def step():
        B.nvfp4_fp8_quantize_rows(xbuf, qx, sx)
        B.nvfp4_fp8_gemm(qx, sx, qw, sw, out=y)

    xbuf.copy_(dev_bf16(wl.random_activation_bits(m, k, seed=30)))
    graph = capture(step)
    for seed in (32, 33, 34):
        x = wl.random_activation_bits(m, k, seed=seed)
        xbuf.copy_(dev_bf16(x))
        graph.replay()
        torch.cuda.synchronize()
        got_q, got_s, got_y = qx.view(torch.uint8).cpu().numpy(), sx.cpu().numpy(), host_bits(y)
        oq, os_ = F.quantize_rows(x)
        assert np.array_equal(got_q, oq) and np.array_equal(got_s.view(np.uint32), os_.view(np.uint32))
        eq, es = B.nvfp4_fp8_quantize_rows(dev_bf16(x))
        ey = host_bits(B.nvfp4_fp8_gemm(eq, es, qw, sw))
        assert np.array_equal(got_y, ey), f"replay {seed} differs from the eager GEMM"


def test_w4a4_graph_replays():
    n, k, m = 1027, 512, 8
    w = wl.random_weight_bits(n, k, sigma=0.02, seed=41)
    pw, sw, gw = B.nvfp4_quantize(dev_bf16(w))
    gi = torch.tensor(np.float32(2.0 ** -7), device=DEV)
    xbuf = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((int(B.load_library().nvfp4_w4a4_workspace_bytes(m, k)),), dtype=torch.uint8, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    held = {}

    def step():
        xp, xs = B.nvfp4_quantize_activations(xbuf, gi)
        held["xp"], held["xs"] = xp, xs
        B.nvfp4_w4a4_gemm(xp, xs, gi, pw, sw, gw, out=y, workspace=ws)

    xbuf.copy_(dev_bf16(wl.random_activation_bits(m, k, seed=40)))
    graph = capture(step)
    for seed in (42, 43, 44):
        x = wl.random_activation_bits(m, k, seed=seed)
        xbuf.copy_(dev_bf16(x))
        graph.replay()
        torch.cuda.synchronize()
        op, os_ = A.quantize_activations(x, np.float32(2.0 ** -7))
        assert np.array_equal(held["xp"].cpu().numpy(), op)
        assert np.array_equal(held["xs"].view(torch.uint8).cpu().numpy(), os_)
        exp, exs = B.nvfp4_quantize_activations(dev_bf16(x), gi)
        ey = host_bits(B.nvfp4_w4a4_gemm(exp, exs, gi, pw, sw, gw))
        assert np.array_equal(host_bits(y), ey), f"replay {seed} differs from the eager GEMM"


def test_import_graph_replays():
    n, k = 300, 256
    rng = np.random.default_rng(50)
    part = torch.tensor(np.float32([1e-3, 2e-3]), device=DEV)
    sbuf = torch.zeros((n, k // 16), dtype=torch.uint8, device=DEV)
    gs = torch.empty((), dtype=torch.float32, device=DEV)
    flags = torch.empty((), dtype=torch.int32, device=DEV)
    graph = capture(lambda: B.nvfp4_import_checkpoint(part, sbuf, k, "compressed-tensors", gs, flags))
    for plant in (None, (0, 0), (n - 1, k // 16 - 1), None):
        s = rng.integers(0, 0x7F, size=(n, k // 16)).astype(np.uint8)
        if plant is not None:
            s[plant] = 0xFF
        sbuf.copy_(dev_u8(s))
        graph.replay()
        torch.cuda.synchronize()
        want_gs, want_f = I.import_report(part.cpu().numpy(), s, I.COMPRESSED_TENSORS)
        assert f32_bits(gs.item()) == f32_bits(want_gs) and int(flags.item()) == want_f


def test_moe_forward_graph_replays_with_new_routing():
    """The expert layer holds no host synchronisation (routing runs on the
    device), so one captured forward replays with new activations, new ids
    and new routing weights written into the captured buffers; every replay
    equals the eager layer bit for bit (the kernels are deterministic)."""
    import oracle.nvfp4_oracle as O

    E, H, I, T, topk = 6, 512, 256, 12, 2
    experts = []
    for rows, k, s0 in ((2 * I, H, 10), (H, I, 1000)):
        bits = wl.moe_expert_bits(rows, k, E, 0.02, 77, s0)
        qs = [O.quantize(bits[e]) for e in range(E)]
        experts.append((dev_u8(np.stack([q[0] for q in qs])), dev_u8(np.stack([q[1] for q in qs])),
                        torch.tensor(np.array([q[2] for q in qs], np.float32), device=DEV)))
    w13, w2 = experts
    xbuf = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, topk), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, topk), dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((int(B.load_library().nvfp4_moe_workspace_bytes(T, topk, E, H, I)),), dtype=torch.uint8,
                     device=DEV)

    def load(seed):
        xbuf.copy_(dev_bf16(wl.random_activation_bits(T, H, seed=seed)))
        i, w = wl.moe_routing(T, E, topk, seed)
        ids.copy_(torch.from_numpy(i))
        tw.copy_(torch.from_numpy(w))

    load(40)
    graph = capture(lambda: B.nvfp4_moe_w4a16_forward(xbuf, ids, tw, w13, w2, out=out, workspace=ws))
    for seed in (41, 42, 43):
        load(seed)
        graph.replay()
        torch.cuda.synchronize()
        got = host_bits(out)
        eager = host_bits(B.nvfp4_moe_w4a16_forward(xbuf.clone(), ids.clone(), tw.clone(), w13, w2))
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), f"replay {seed} differs from the eager layer"
