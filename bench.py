#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A16 lm_head hot path on one MI355X.

One step = one pass of the whole path over the workload's synthetic inputs:
an in-place NVFP4 re-quantization of the bf16 lm_head weight
(nvfp4_refresh_inplace: amax, global scale, block scales, codes, packing)
followed by the W4A16 GEMM at every activation row count M of the workload.
Inputs are resident in HBM before timing starts.  Three copies of the
quantized weight rotate so that every GEMM reads weights that were not just
touched (the 8B-shape weights, 296 MB, would otherwise partly hit the
256 MB last-level cache).

Prints one JSON line: value = algorithmic bytes of the step / step time
(TB/s), plus per-operation rates, the roofline of the dominant operation and
the CPU oracle timed on a bounded sample.  After the step, the prefill GEMM of
the Qwen-shaped workload (151936 x 5120, M = 4096) is timed on its own and
reported in per_op with its MFMA roofline (the TFLOP/s half of the metric).
The SHA-256 of every input tensor and the oracle host's CPUs are recorded.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 W4A16 lm_head GEMM: HBM TB/s at M=1..64, TFLOP/s at M=4096; quant GB/s"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA


def quant_bytes(n: int, k: int) -> float:
    """Read W twice (amax, encode), write codes (0.5 B) and scales (1/16 B) per weight."""
    return n * k * (2 + 2 + 0.5 + 0.0625)


def gemm_bytes(m: int, n: int, k: int) -> float:
    return n * k * (0.5 + 0.0625) + 2 * m * k + 2 * m * n + 4


def gemm_flops(m: int, n: int, k: int) -> float:
    return 2.0 * m * n * k


def decode_kernel_name(m: int, k: int) -> str:
    """Which decode kernel the library dispatches for (M, K) (mirrors its
    dispatch rule, for N up to 262144)."""
    if k % 32 == 0 and ((m == 1 and k <= 8192) or (m == 2 and k <= 4096)):
        return "gemv_dot_kernel"
    if k % 256 != 0:
        return "gemv_mfma_ragged_kernel"
    if 3 <= m <= 16:
        fits = lambda cols, nw, depth: m * (2 * cols + 16) + nw * (2048 * max(depth, 1) + 1024) + 64 <= 160 * 1024
        deep = k % 1024 == 0
        if (deep and (fits(k, 8, 2) or fits(k, 16, 2))) or fits(k, 16, 0) or (not deep and fits(k, 8, 0)):
            return "gemv_xres_kernel"
        if any(k % np_ == 0 and (k // np_) % 1024 == 0 and fits(k // np_, 16, 2) for np_ in (2, 4, 8)):
            return "gemv_xphase_kernel"
    return "gemv_panel_kernel" if k % 512 == 0 else "gemv_mfma_kernel"


class TimingEvent:
    """A HIP event for timing only, used like torch.cuda.Event(enable_timing=True).

    It is created with hipEventDisableSystemFence: a default event is recorded
    with a system-scope release (cache write-back and invalidate), which puts a
    ~6 us bubble between the kernels it separates and slows the one after it.
    These events only time work, so they skip the fence; read them after
    torch.cuda.synchronize().  The HIP runtime is the one already loaded in
    the process (torch's)."""

    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes

            path = None
            with open("/proc/self/maps") as fh:
                for line in fh:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes

        self._h = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._h), self._DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self) -> None:
        import ctypes

        import torch

        rc = self._lib().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes

        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def __del__(self):
        # through the instance's class: at interpreter shutdown the module's
        # globals (this class's name included) may already be None
        hip = getattr(type(self), "_hip", None)
        if getattr(self, "_h", None) is not None and self._h.value and hip is not None:
            hip.hipEventDestroy(self._h)
            self._h = None


def sha256_bits(a) -> str:
    """SHA-256 of an input tensor's bytes (bf16 bit patterns, row-major)."""
    import numpy as np

    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def host_info() -> dict:
    """The host the oracle runs on: logical CPUs, the ones this process may
    use, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count() or 1, "usable_cpus": usable, "cpu_model": model}


def bench_prefill(args, dev, to_dev):
    """The prefill GEMM of the Qwen-shaped workload (151936 x 5120, M = 4096),
    timed outside the step: quantize once, then the GEMM per call with HIP
    events on the stream it is launched on."""
    import numpy as np
    import torch

    from nvfp4_w4a16_lm_amd import binding as B
    from nvfp4_w4a16_lm_amd import workloads as wl

    pw = wl.WORKLOADS[args.prefill_workload]
    t0 = time.perf_counter()
    pb = wl.weight_bits(pw)
    px = wl.activation_bits(pw)
    m = max(pw.ms)
    inputs = {f"{pw.name}/W": sha256_bits(pb), f"{pw.name}/x": sha256_bits(px[:m])}
    print(f"# prefill inputs generated and hashed in {time.perf_counter() - t0:.1f} s: W {pw.n}x{pw.k}, "
          f"x {m}x{pw.k}", file=sys.stderr, flush=True)
    W = to_dev(pb)
    del pb
    X = to_dev(px[:m])
    q = B.nvfp4_quantize(W)
    del W
    Y = torch.empty((m, pw.n), dtype=torch.bfloat16, device=dev)
    # The GPU's clock climbs over the first few back-to-back calls of this
    # MFMA-bound kernel (about 5.9, 5.3, 5.0, 4.8 ms, then flat): warm up
    # for at least 20 calls (~0.1 s) so that the timed calls see the steady
    # clock.
    for _ in range(max(20, args.warmup)):
        B.nvfp4_w4a16_gemm(X, *q, out=Y)
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.prefill_steps):
        a = TimingEvent()
        b = TimingEvent()
        a.record()
        B.nvfp4_w4a16_gemm(X, *q, out=Y)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(np.mean(t))
    achieved = gemm_flops(m, pw.n, pw.k) / (ms * 1e-3) / 1e12
    rec = {"ms": ms, "ms_min": float(np.min(t)), "ms_p50": float(np.median(t)), "ms_p90": float(np.percentile(t, 90)),
           "TFLOP/s": achieved, "TB/s": gemm_bytes(m, pw.n, pw.k) / (ms * 1e-3) / 1e12,
           "calls": int(args.prefill_steps), "in_step": False,
           "shape": {"N": pw.n, "K": pw.k, "M": m},
           "roofline": {"op": f"nvfp4_w4a16_gemm M={m} ({pw.name})", "kernels": "gemm_prefill_kernel",
                        "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / BF16_PEAK_TFLOPS, "traffic": load_traffic(pw.name, f"gemm_m{m}")}}
    del q, X, Y
    torch.cuda.synchronize()
    return f"prefill_{pw.name}_m{m}", rec, inputs


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_w4a16_lm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, op: str):
    """HBM bytes per launch of ``op`` (FETCH_SIZE and WRITE_SIZE counter runs,
    scaled by a plain-copy calibration; profiles/hbm_traffic.md), or None when
    the kernels have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("ops", {}).get(f"{workload}/{op}")


def cpu_baseline(wl, w, w_bits, x_bits, ms, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same step: the first
    ``rows`` weight rows, sized from a short calibration run so that the timed
    sample takes about ``budget_s`` seconds of CPU work."""
    import numpy as np

    import oracle.nvfp4_oracle as O

    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:   # threadpoolctl missing: numpy elementwise work is single-threaded
        blas = 1

    def step(rows):
        sub = np.ascontiguousarray(w_bits[:rows])
        t0 = time.perf_counter()
        gs = O.global_scale(O.weight_amax(sub))
        packed, scales = O.quantize_rows(sub, gs)
        for m in ms:
            O.gemm_ref(x_bits[:m], packed, scales, gs)
        return time.perf_counter() - t0

    probe = min(1024, w.n)
    rate = probe / max(step(probe), 1e-6)                 # rows per second
    rows = int(min(w.n, max(probe, rate * budget_s)))
    dt = step(rows)
    nbytes = quant_bytes(rows, w.k) + sum(gemm_bytes(m, rows, w.k) for m in ms)
    return {
        "value": nbytes / dt / 1e12,
        "unit": "TB/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"{rows} of {w.n} weight rows ({w.k} columns): amax + quantize, then fp64 GEMM at "
                   f"M={list(ms)}; {dt:.1f} s; numpy elementwise on 1 thread, BLAS on {blas}"),
        **host_info(),
    }


def moe_cpu_baseline(mw, w13_bits, w2_bits, x_bits, budget_s: float):
    """The oracle's whole expert layer, as it stands, on a bounded sample of
    the workload: the intermediate dimension cut to its first ``i_s`` columns
    (w13 rows [0, i_s) and [I, I + i_s), w2 columns [0, i_s)), every expert
    and every token count, sized from a short calibration run to about
    ``budget_s`` seconds.  The experts are quantized by the oracle first
    (not timed)."""
    import numpy as np

    import oracle.nvfp4_oracle as O
    import oracle.nvfp4_moe_oracle as MO
    from nvfp4_w4a16_lm_amd import workloads as wl

    E, H, I, topk = mw.experts, mw.hidden, mw.inter, mw.topk

    def quant(bits):
        qs = [O.quantize(bits[e]) for e in range(E)]
        return (np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]),
                np.array([q[2] for q in qs], dtype=np.float32))

    def layer(i_s):
        w13 = quant(np.concatenate([w13_bits[:, :i_s], w13_bits[:, I:I + i_s]], axis=1))
        w2 = quant(np.ascontiguousarray(w2_bits[:, :, :i_s]))
        t0 = time.perf_counter()
        nbytes = 0.0
        for T in mw.tokens:
            ids, tw = wl.moe_routing(T, E, topk, mw.cfg)
            MO.moe_ref(x_bits[:T], ids, tw, w13, w2)
            b13, b2 = moe_active_bytes(ids, E, H, i_s)
            nbytes += b13 + b2 + 4 * T * H
        return time.perf_counter() - t0, nbytes

    probe = 64
    dt, _ = layer(probe)
    i_s = int(min(I, max(probe, probe * budget_s / max(dt, 1e-6))) // 16 * 16)
    dt, nbytes = layer(i_s)
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    return {"value": nbytes / dt / 1e12, "unit": "TB/s", "cores": int(blas), "kind": "oracle",
            "sample": (f"intermediate dimension {i_s} of {I} (all {E} experts, H {H}), T = {list(mw.tokens)}: "
                       f"the fp64 layer; {dt:.1f} s; numpy elementwise on 1 thread, BLAS on {blas}"),
            **host_info()}


def moe_active_bytes(ids, E: int, H: int, I: int):
    """NVFP4 bytes of the experts that receive at least one pair: (w13, w2)."""
    import numpy as np

    active = int(np.unique(ids).size)
    return active * 2 * I * H * (0.5 + 0.0625), active * H * I * (0.5 + 0.0625)


def bench_moe(args, mw, dev) -> int:
    """The W4A16 expert layer (routing, grouped GEMM with w13, SiLU-and-mul,
    grouped GEMM with w2, weighted combine) at each token count of the
    workload.  value = algorithmic HBM bytes of the layer over its time: the
    NVFP4 bytes of the experts that receive a pair, x, the bf16 intermediates
    written and read once, and the output."""
    import numpy as np
    import torch

    from nvfp4_w4a16_lm_amd import binding as B
    from nvfp4_w4a16_lm_amd import workloads as wl

    E, H, I, topk = mw.experts, mw.hidden, mw.inter, mw.topk
    t0 = time.perf_counter()
    w13_bits = wl.moe_expert_bits(2 * I, H, E, mw.sigma, mw.cfg, 10)
    w2_bits = wl.moe_expert_bits(H, I, E, mw.sigma, mw.cfg, 1000)
    tmax = max(mw.tokens)
    x_bits = wl.normal_bits(tmax, H, 1.0, (mw.cfg, 2))
    print(f"# MoE inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def quant_experts(bits, rows, k):
        packed = torch.empty((E, rows, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((E, rows, k // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty((E,), dtype=torch.float32, device=dev)
        for e in range(E):
            we = to_dev(bits[e])
            B.nvfp4_refresh_inplace(we, packed[e], scales[e], gs[e])
            del we
        return packed, scales, gs

    w13 = quant_experts(w13_bits, 2 * I, H)
    w2 = quant_experts(w2_bits, H, I)
    X = to_dev(x_bits)
    torch.cuda.synchronize()
    per_t = {}
    for T in mw.tokens:
        ids_np, tw_np = wl.moe_routing(T, E, topk, mw.cfg)
        ids = torch.from_numpy(ids_np).to(dev)
        tw = torch.from_numpy(tw_np).to(dev)
        x = X[:T]
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((int(B.load_library().nvfp4_moe_workspace_bytes(T, topk, E, H, I)),), dtype=torch.uint8,
                         device=dev)
        h = torch.empty((T * topk, 2 * I), dtype=torch.bfloat16, device=dev)
        gws = torch.empty((int(B.load_library().nvfp4_moe_gemm_workspace_bytes(T * topk, E)) + 16,),
                          dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            B.nvfp4_moe_w4a16_forward(x, ids, tw, w13, w2, out=out, workspace=ws)
        torch.cuda.synchronize()
        evf, evg = [], []
        for _ in range(args.steps):
            a = TimingEvent()
            b = TimingEvent()
            c = TimingEvent()
            a.record()
            B.nvfp4_moe_w4a16_forward(x, ids, tw, w13, w2, out=out, workspace=ws)
            b.record()
            B.nvfp4_moe_w4a16_gemm(x, ids, topk, *w13, out=h, workspace=gws)
            c.record()
            evf.append((a, b))
            evg.append((b, c))
        torch.cuda.synchronize()
        tf = float(np.mean([a.elapsed_time(b) for a, b in evf]))
        tg = float(np.mean([a.elapsed_time(b) for a, b in evg]))
        b13, b2 = moe_active_bytes(ids_np, E, H, I)
        P = T * topk
        layer_bytes = b13 + b2 + 2 * T * H + 2 * P * (2 * I) * 2 + 2 * P * I * 2 + 2 * P * H * 2 + 2 * T * H
        g1_bytes = b13 + 2 * T * H + 2 * P * 2 * I
        per_t[T] = {"ms": tf, "TB/s": layer_bytes / (tf * 1e-3) / 1e12, "bytes": layer_bytes,
                    "experts_active": int(np.unique(ids_np).size),
                    "grouped_gemm_w13_ms": tg, "grouped_gemm_w13_TB/s": g1_bytes / (tg * 1e-3) / 1e12,
                    "grouped_gemm_w13_bytes": g1_bytes}
    total_bytes = sum(v["bytes"] for v in per_t.values())
    total_ms = sum(v["ms"] for v in per_t.values())
    tdom = max(per_t, key=lambda t: per_t[t]["grouped_gemm_w13_ms"])
    ach = per_t[tdom]["grouped_gemm_w13_bytes"] / (per_t[tdom]["grouped_gemm_w13_ms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": total_bytes / (total_ms * 1e-3) / 1e12,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x nvfp4 (fp32 accumulate)",
        "data": "synthetic (seeded; no trained weights)",
        "config": {"workload": mw.name, "description": mw.description, "E": E, "H": H, "I": I, "topk": topk,
                   "T": list(mw.tokens), "step": "nvfp4_moe_w4a16_forward at each T"},
        "per_op": {f"moe_forward_t{t}": v for t, v in per_t.items()},
        "roofline": {"op": f"nvfp4_moe_w4a16_gemm (w13) T={tdom}",
                     "kernels": "moe_route + the expert kernels of each pair-count class",
                     "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBPS, "traffic": None},
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = moe_cpu_baseline(mw, w13_bits, w2_bits, x_bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b",
                    help="llama3_8b (default), llama3_70b, qwen_prefill, heavy_tail, tiny; "
                         "moe_8x4096 / moe_small time the W4A16 expert layer instead")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=3, help="rotating quantized-weight copies")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    ap.add_argument("--prefill-workload", default="qwen_prefill",
                    help="workload whose prefill GEMM is timed after the step (its largest M)")
    ap.add_argument("--prefill-steps", type=int, default=10, help="timed prefill GEMM calls")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill GEMM timing")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported (the path shards by "
              "vocabulary rows; each GPU would run this same benchmark on its shard).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from nvfp4_w4a16_lm_amd import binding as B
    from nvfp4_w4a16_lm_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_probe:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch, 5 launches
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_launch": src.numel() * 4, "launches": 5}))
        return 0
    B.load_library()
    dev = torch.device("cuda:0")
    if args.workload in wl.MOE_WORKLOADS:
        return bench_moe(args, wl.MOE_WORKLOADS[args.workload], dev)
    w = wl.WORKLOADS[args.workload]
    n, k, ms = w.n, w.k, w.ms
    t0 = time.perf_counter()
    w_bits = wl.weight_bits(w)
    x_bits = wl.activation_bits(w)
    print(f"# inputs generated in {time.perf_counter() - t0:.1f} s: W {n}x{k}, x {x_bits.shape}",
          file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    inputs = {f"{w.name}/W": sha256_bits(w_bits), f"{w.name}/x": sha256_bits(x_bits)}
    W = to_dev(w_bits)
    X = to_dev(x_bits)
    copies = max(1, args.copies)
    Q = [B.nvfp4_quantize(W) for _ in range(copies)]
    Y = {m: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for m in ms}
    xs = {m: X[:m] for m in ms}
    torch.cuda.synchronize()

    ops = ["quantize"] + [f"gemm_m{m}" for m in ms]
    ev = {op: [] for op in ops}

    def step(i: int, record: bool):
        qi = i % copies
        e0 = TimingEvent() if record else None
        if record:
            e0.record()
        B.nvfp4_refresh_inplace(W, *Q[qi])
        if record:
            e1 = TimingEvent()
            e1.record()
            ev["quantize"].append((e0, e1))
            e0 = e1
        for j, m in enumerate(ms):
            qj = (qi + 1 + j % max(1, copies - 1)) % copies if copies > 1 else 0
            B.nvfp4_w4a16_gemm(xs[m], *Q[qj], out=Y[m])
            if record:
                e1 = TimingEvent()
                e1.record()
                ev[f"gemm_m{m}"].append((e0, e1))
                e0 = e1

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # the per-operation events inside the timed steps are fence-free
    # (TimingEvent); the bracket around them is an ordinary event pair
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, True)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    avg_ms = {op: float(np.mean([a.elapsed_time(b) for a, b in ev[op]])) for op in ops}
    # spread of the per-call times: min, median, 90th percentile
    spread = {op: {"ms_min": float(np.min(t)), "ms_p50": float(np.median(t)), "ms_p90": float(np.percentile(t, 90))}
              for op in ops for t in [[a.elapsed_time(b) for a, b in ev[op]]]}

    # Pre-quantized checkpoint import (not part of the step): global scale from
    # the partition scales + one NaN scan of the block scales, timed the same way.
    ps = Q[0][2].reshape(1).clone()
    gsi = torch.empty((), dtype=torch.float32, device=dev)
    flg = torch.empty((), dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        B.nvfp4_import_checkpoint(ps, Q[i % copies][1], k, "modelopt", gsi, flg)
    torch.cuda.synchronize()
    imp_ev = []
    for i in range(args.steps):
        a = TimingEvent()
        b = TimingEvent()
        a.record()
        B.nvfp4_import_checkpoint(ps, Q[i % copies][1], k, "modelopt", gsi, flg)
        b.record()
        imp_ev.append((a, b))
    torch.cuda.synchronize()
    if int(flg.item()) != 0:
        raise RuntimeError(f"checkpoint import flags {int(flg.item())} on freshly quantized scales")
    imp_ms = float(np.mean([a.elapsed_time(b) for a, b in imp_ev]))
    imp_bytes = n * k / 16 + 4 + 8

    # The FP8 copy (not part of the step): row-wise E4M3 quantization of the
    # weight, then per M the per-token activation quantization + FP8 GEMM.
    fq, fs = B.nvfp4_fp8_quantize_rows(W)
    xq8 = {m: B.nvfp4_fp8_quantize_rows(xs[m]) for m in ms}
    y8 = {m: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for m in ms}
    fp8_ev = {"fp8_quantize_w": []} | {f"fp8_linear_m{m}": [] for m in ms}

    def fp8_step(record: bool):
        e0 = TimingEvent() if record else None
        if record:
            e0.record()
        B.nvfp4_fp8_quantize_rows(W, fq, fs)
        for m in ms:
            if record:
                e1 = TimingEvent()
                e1.record()
                fp8_ev["fp8_quantize_w" if m == ms[0] else f"fp8_linear_m{prev}"].append((e0, e1))
                e0 = e1
            B.nvfp4_fp8_quantize_rows(xs[m], *xq8[m])
            B.nvfp4_fp8_gemm(*xq8[m], fq, fs, out=y8[m])
            prev = m
        if record:
            e1 = TimingEvent()
            e1.record()
            fp8_ev[f"fp8_linear_m{prev}"].append((e0, e1))

    for _ in range(args.warmup):
        fp8_step(False)
    for _ in range(args.steps):
        fp8_step(True)
    torch.cuda.synchronize()
    fp8_ms = {op: float(np.mean([a.elapsed_time(b) for a, b in v])) for op, v in fp8_ev.items()}

    # NVFP4 W4A4 (not part of the step): per M, activation quantization with a
    # static global input scale + the W4A4 GEMM on the step's quantized weight.
    gi = torch.tensor(np.float32(2.0 ** -7), device=dev)
    wsp = torch.empty((int(B.load_library().nvfp4_w4a4_workspace_bytes(max(ms), k)),), dtype=torch.uint8,
                      device=dev)
    w4_ev = {m: [] for m in ms}
    for it in range(args.warmup + args.steps):
        for m in ms:
            a = TimingEvent()
            b = TimingEvent()
            a.record()
            xp4, xs4 = B.nvfp4_quantize_activations(xs[m], gi)
            B.nvfp4_w4a4_gemm(xp4, xs4, gi, *Q[0], out=Y[m], workspace=wsp)
            b.record()
            if it >= args.warmup:
                w4_ev[m].append((a, b))
    torch.cuda.synchronize()
    w4_ms = {m: float(np.mean([a.elapsed_time(b) for a, b in v])) for m, v in w4_ev.items()}

    step_bytes = quant_bytes(n, k) + sum(gemm_bytes(m, n, k) for m in ms)
    value = step_bytes / (ms_per_step * 1e-3) / 1e12

    prefill = None
    if not args.no_prefill and args.prefill_workload != w.name:
        prefill = bench_prefill(args, dev, to_dev)
        inputs.update(prefill[2])

    per_op = {"quantize": {"ms": avg_ms["quantize"], **spread["quantize"],
                           "GB/s": quant_bytes(n, k) / (avg_ms["quantize"] * 1e-3) / 1e9}}
    per_op["import_checkpoint"] = {"ms": imp_ms, "GB/s": imp_bytes / (imp_ms * 1e-3) / 1e9,
                                   "kernels": "import_prepare (1 wavefront) + scale_nan_scan",
                                   "in_step": False}
    per_op["fp8_quantize_w"] = {"ms": fp8_ms["fp8_quantize_w"],
                                "GB/s": (n * k * 3 + 4 * n) / (fp8_ms["fp8_quantize_w"] * 1e-3) / 1e9,
                                "kernels": "fp8_quant_rows (bf16 weight -> e4m3 + per-row scales)",
                                "in_step": False}
    for m in ms:
        t8 = fp8_ms[f"fp8_linear_m{m}"] * 1e-3
        per_op[f"fp8_linear_m{m}"] = {"ms": fp8_ms[f"fp8_linear_m{m}"],
                                      "TB/s": (n * k + 4 * n + 3 * m * k + 4 * m + 2 * m * n) / t8 / 1e12,
                                      "TFLOP/s": gemm_flops(m, n, k) / t8 / 1e12,
                                      "kernels": "fp8_quant_rows (per token) + fp8_gemm", "in_step": False}
    for m in ms:
        t4 = w4_ms[m] * 1e-3
        per_op[f"w4a4_m{m}"] = {"ms": w4_ms[m], "TB/s": gemm_bytes(m, n, k) / t4 / 1e12,
                                "TFLOP/s": gemm_flops(m, n, k) / t4 / 1e12,
                                "kernels": "quant_pack (activations, given scale) + w4a4_dequant_x + the W4A16 GEMM",
                                "in_step": False}
    for m in ms:
        t = avg_ms[f"gemm_m{m}"] * 1e-3
        per_op[f"gemm_m{m}"] = {"ms": avg_ms[f"gemm_m{m}"], **spread[f"gemm_m{m}"],
                                "TB/s": gemm_bytes(m, n, k) / t / 1e12,
                                "TFLOP/s": gemm_flops(m, n, k) / t / 1e12}

    if prefill is not None:
        per_op[prefill[0]] = prefill[1]

    dom = max(ops, key=lambda op: avg_ms[op])
    if dom == "quantize":
        achieved = quant_bytes(n, k) / (avg_ms[dom] * 1e-3) / 1e9
        roof = {"op": "nvfp4_refresh_inplace",
                "kernels": "amax_init (1 thread) + amax + quant_pack, back to back on one stream",
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(w.name, "quantize")}
    else:
        m = int(dom.split("_m")[1])
        if m > 64:
            achieved = gemm_flops(m, n, k) / (avg_ms[dom] * 1e-3) / 1e12
            roof = {"op": f"nvfp4_w4a16_gemm M={m}", "kernels": "gemm_prefill_kernel", "bound": "mfma",
                    "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS, "traffic": load_traffic(w.name, dom)}
        else:
            achieved = gemm_bytes(m, n, k) / (avg_ms[dom] * 1e-3) / 1e9
            roof = {"op": f"nvfp4_w4a16_gemm M={m}", "kernels": decode_kernel_name(m, k), "bound": "hbm",
                    "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(w.name, dom)}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x nvfp4 (fp32 accumulate)",
        "data": "synthetic (seeded; no trained weights)",
        "config": {"workload": w.name, "description": w.description, "N": n, "K": k, "M": list(ms),
                   "step": "nvfp4_refresh_inplace + nvfp4_w4a16_gemm at each M", "weight_copies": copies},
        "per_op": per_op,
        "roofline": roof,
        "inputs_sha256": inputs,
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, w, w_bits, x_bits, ms, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
