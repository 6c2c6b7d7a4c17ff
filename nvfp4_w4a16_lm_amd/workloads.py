"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module creates bf16 tensors (as uint16 bit arrays) of the lm_head shapes
and value distributions the workloads use.  It holds none of the method's
arithmetic: no scale, no rounding to E2M1/E4M3, no dequantization.  Its one
numeric step is rounding float32 draws to bf16 (round to nearest even), which
is how the synthetic weights and activations come into existence.

Recipe (numpy PCG64 ``default_rng``):

* Tensors are generated in row chunks of ``max(1, CHUNK_ELEMS // K)`` rows;
  chunk ``c`` of stream ``s`` of config ``cfg`` draws from
  ``default_rng([cfg, s, c])`` (independent chunks, generated on a thread
  pool).  The tiny weight is one chunk drawn from ``default_rng(0)``.
  Streams: 0 = weight, 1 = outlier mask, 2 = activations, 3 = refresh noise,
  4 = bias.
* Normal draws are float32 ``standard_normal`` multiplied by the float32
  standard deviation, then rounded to bf16.
* Llama-3-8B shape: exactly ``round(0.001 * N * K)`` distinct positions, drawn
  with ``choice(N * K, count, replace=False)``, are multiplied by 20 before the
  bf16 rounding.
* Heavy-tailed: ``0.01 * standard_t(3)`` drawn in float64, rounded to float32
  then bf16; row 0 is all zero; row N-1 repeats a pattern of E2M1 grid values
  in which every 16-block holds +-6 and both +0 and -0.
* 70B refresh: ``W' = bf16(float32(W) + 1e-3 * standard_normal)``.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np
import torch

CHUNK_ELEMS = 1 << 23
_THREADS = max(1, min(16, os.cpu_count() or 1))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int            # seed namespace
    n: int              # vocab rows
    k: int              # hidden size
    sigma: float        # weight standard deviation
    ms: tuple           # activation row counts measured
    m_draw: int         # activation rows drawn (x[:m] is used for each m)
    kind: str = "normal"   # "normal" | "outliers" | "heavy"
    description: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1024, 512, 0.02, (4,), 4,
                     description="weight 1024x512 N(0,0.02) seed 0; x 4x512 N(0,1)"),
    "llama3_8b": Workload("llama3_8b", 2, 128256, 4096, 0.02, (1, 8, 32, 64), 64, "outliers",
                          description="lm_head 128256x4096 N(0,0.02) + 0.1% entries x20; "
                                      "decode M in {1,8,32,64}"),
    "llama3_70b": Workload("llama3_70b", 3, 128256, 8192, 0.015, (1, 16, 64), 64,
                           description="lm_head 128256x8192 N(0,0.015); M in {1,16,64}; "
                                       "refresh after N(0,1e-3) noise"),
    "qwen_prefill": Workload("qwen_prefill", 4, 151936, 5120, 0.02, (4096,), 4096,
                             description="lm_head 151936x5120 N(0,0.02); prefill M=4096"),
    "heavy_tail": Workload("heavy_tail", 5, 129280, 7168, 0.01, (1, 8192), 8192, "heavy",
                           description="lm_head 129280x7168 0.01*t(3), zero row 0, "
                                       "E2M1-grid row N-1; M=1 and M=8192"),
}


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def chunk_rows(k: int) -> int:
    return max(1, CHUNK_ELEMS // k)


def _chunked(n: int, k: int, fill) -> np.ndarray:
    """Run ``fill(chunk_index, r0, r1) -> uint16 [r1-r0, k]`` over row chunks in threads."""
    out = np.empty((n, k), dtype=np.uint16)
    rows = chunk_rows(k)
    starts = list(range(0, n, rows))

    def work(ci):
        r0 = starts[ci]
        r1 = min(n, r0 + rows)
        out[r0:r1] = fill(ci, r0, r1)

    if len(starts) == 1:
        work(0)
    else:
        with concurrent.futures.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def normal_bits(n: int, k: int, sigma: float, seed: tuple) -> np.ndarray:
    """bf16 bits of ``sigma * N(0,1)`` float32 draws; chunk c uses default_rng([*seed, c])."""
    s = np.float32(sigma)

    def fill(ci, r0, r1):
        rng = np.random.default_rng([*seed, ci])
        return f32_to_bf16_bits(rng.standard_normal((r1 - r0, k), dtype=np.float32) * s)

    return _chunked(n, k, fill)


def weight_bits(w: Workload) -> np.ndarray:
    """The workload's bf16 weight [N, K] as uint16 bits."""
    if w.kind == "heavy":
        return _heavy_weight(w)
    if w.name == "tiny":
        f = np.random.default_rng(0).standard_normal((w.n, w.k), dtype=np.float32) * np.float32(w.sigma)
        return f32_to_bf16_bits(f)
    if w.kind != "outliers":
        return normal_bits(w.n, w.k, w.sigma, (w.cfg, 0))
    count = int(round(0.001 * w.n * w.k))
    pos = np.sort(np.random.default_rng([w.cfg, 1]).choice(w.n * w.k, size=count, replace=False))
    s = np.float32(w.sigma)

    def fill(ci, r0, r1):
        f = np.random.default_rng([w.cfg, 0, ci]).standard_normal((r1 - r0, w.k), dtype=np.float32) * s
        lo, hi = np.searchsorted(pos, [r0 * w.k, r1 * w.k])
        flat = f.reshape(-1)
        flat[pos[lo:hi] - r0 * w.k] *= np.float32(20.0)
        return f32_to_bf16_bits(f)

    return _chunked(w.n, w.k, fill)


def grid_row_bits(k: int) -> np.ndarray:
    """Row of E2M1 grid values: +G[k%8] for k%16 < 8, else -G[k%8] (with -0.0)."""
    g = np.array([6.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 0.0], dtype=np.float32)
    idx = np.arange(k)
    vals = g[idx % 8]
    vals = np.where(idx % 16 < 8, vals, -vals).astype(np.float32)
    return f32_to_bf16_bits(vals)


def _heavy_weight(w: Workload) -> np.ndarray:
    def fill(ci, r0, r1):
        t = np.random.default_rng([w.cfg, 0, ci]).standard_t(3, size=(r1 - r0, w.k)) * w.sigma
        return f32_to_bf16_bits(t.astype(np.float32))

    out = _chunked(w.n, w.k, fill)
    out[0] = 0
    out[w.n - 1] = grid_row_bits(w.k)
    return out


def activation_bits(w: Workload, m: int | None = None) -> np.ndarray:
    """bf16 activations x[:m] of the workload's N(0,1) draw [m_draw, K]."""
    x = normal_bits(w.m_draw, w.k, 1.0, (w.cfg, 2))
    return x if m is None else x[:m]


def refresh_weight_bits(w: Workload, w_bits: np.ndarray, sigma: float = 1e-3) -> np.ndarray:
    """``bf16(float32(W) + sigma * N(0,1))`` for the in-place refresh workload."""
    s = np.float32(sigma)
    k = w_bits.shape[1]

    def fill(ci, r0, r1):
        noise = np.random.default_rng([w.cfg, 3, ci]).standard_normal((r1 - r0, k), dtype=np.float32) * s
        return f32_to_bf16_bits(bf16_bits_to_f32(w_bits[r0:r1]) + noise)

    return _chunked(w_bits.shape[0], k, fill)


def bias_bits(n: int, seed: int = 0, sigma: float = 1.0) -> np.ndarray:
    return normal_bits(1, n, sigma, (seed, 4))[0]


def random_weight_bits(n: int, k: int, sigma: float = 0.02, seed: int = 0) -> np.ndarray:
    """Ad-hoc shapes for edge-case tests (ragged N and K, tiny sizes)."""
    return normal_bits(n, k, sigma, (100, seed, n, k))


def random_activation_bits(m: int, k: int, seed: int = 0) -> np.ndarray:
    return normal_bits(m, k, 1.0, (101, seed, m, k))


# ---------------------------------------------------------------------------
# Mixture-of-experts inputs.  Expert e's weights are stream (cfg, 10 + e) for
# w13 and (cfg, 1000 + e) for w2, N(0, sigma); activations stream (cfg, 2);
# routing stream (cfg, 5): each token picks ``topk`` distinct experts
# uniformly (``choice(E, topk, replace=False)``) with weights drawn from
# U(0.1, 1) and divided by their float32 sum.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    name: str
    cfg: int
    experts: int        # E
    hidden: int         # H
    inter: int          # I (w13 has 2I output rows)
    topk: int
    sigma: float
    tokens: tuple       # T values measured
    description: str = ""


MOE_WORKLOADS = {
    "moe_small": MoeWorkload("moe_small", 20, 8, 512, 256, 2, 0.02, (5,),
                             description="8 experts, H 512, I 256, top-2"),
    "moe_8x4096": MoeWorkload("moe_8x4096", 21, 8, 4096, 14336, 2, 0.02, (1, 16, 64),
                              description="8 experts, H 4096, I 14336, top-2; decode T in {1,16,64}"),
}


def moe_expert_bits(rows: int, k: int, experts: int, sigma: float, cfg: int, stream0: int) -> np.ndarray:
    """bf16 bits [E, rows, k]: expert e drawn from stream (cfg, stream0 + e)."""
    out = np.empty((experts, rows, k), dtype=np.uint16)
    for e in range(experts):
        out[e] = normal_bits(rows, k, sigma, (cfg, stream0 + e))
    return out


def moe_routing(tokens: int, experts: int, topk: int, cfg: int) -> tuple[np.ndarray, np.ndarray]:
    """(topk_ids int32 [T, topk], topk_weights float32 [T, topk])."""
    rng = np.random.default_rng([cfg, 5, tokens])
    ids = np.stack([rng.choice(experts, size=topk, replace=False) for _ in range(tokens)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(tokens, topk)).astype(np.float32)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return ids.reshape(tokens, topk), w.reshape(tokens, topk)
