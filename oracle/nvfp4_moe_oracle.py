"""Plain CPU oracle for the NVFP4 W4A16 mixture-of-experts layer: per-expert
NVFP4 weights, bf16 activations, top-k routing.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

Sources (cited by page title and section):

* P2 = vLLM source view of ``vllm/model_executor/layers/quantization/modelopt.py``,
  ``ModelOptNvFp4FusedMoE``: ``use_a16`` for the W4A16 NVFP4 recipe;
  ``create_weights`` lays the experts out as ``w13_weight`` uint8
  ``[E, 2I, H/2]`` with e4m3 ``w13_weight_scale`` ``[E, 2I, H/16]`` and float32
  ``w13_weight_scale_2`` ``[E, 2]`` (one per fused shard), ``w2_weight``
  ``[E, H, I/2]`` with ``w2_weight_scale`` ``[E, H, I/16]`` and
  ``w2_weight_scale_2`` ``[E]``; ``process_weights_after_loading`` keeps one
  global scale for w13, the w1 column, and warns when the w3 column differs;
  ``apply`` takes the activations, ``topk_weights`` and ``topk_ids``.
* P1 = vLLM API docs, ``quantization.online.lm_head``: the NVFP4 format and
  its dequantization (``oracle.nvfp4_oracle``).

Readings (also listed in the repository's design notes):

E1  Routing: pair ``p = t * topk + j`` (token t, slot j) goes to expert
    ``topk_ids[t, j]``.  Experts process their pairs in increasing ``p``; the
    grouping does not change any value.  Ids outside ``[0, E)`` are outside
    the contract (this oracle raises).
E2  Expert GEMM: ``y[p] = x[row(p)] . deq(W_e)^T`` with ``deq`` the NVFP4
    dequantization of P1 using the expert's own global scale; the first GEMM
    reads token ``row(p) = p // topk``, the second reads pair row ``p``.
E3  Activation: the act-and-mul layout ``[w1; w3]`` of ``w13`` (the first I
    output rows gate, the last I rows up), with SiLU:
    ``a = silu(h[:I]) * h[I:]``, ``silu(g) = g / (1 + exp(-g))`` (the pages
    name the activation only through ``layer.activation``; SiLU-and-mul is
    the plain reading of ``is_act_and_mul``).
E4  Combine: ``out[t] = sum_j topk_weights[t, j] * o[t * topk + j]``.
E5  Intermediate precision: the GEMM outputs ``h`` and ``o`` and the
    activation ``a`` are bf16 tensors (one rounding each, as the model dtype
    is bf16); every sum is accumulated in float32 or wider.  The fp64
    reference below carries no intermediate rounding; ``moe_tolerance``
    bounds what those roundings and float32 sums can add.
E6  Global scale of w13: the w1 column of ``w13_weight_scale_2``
    (``collapse_w13_scale2``), flagged when the w3 column differs.
"""

from __future__ import annotations

import numpy as np

from oracle import nvfp4_oracle as O


def route(topk_ids: np.ndarray, num_experts: int) -> tuple[np.ndarray, list[np.ndarray]]:
    """E1: (pairs per expert, the pair indices of each expert in increasing order)."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= num_experts):
        raise O.OracleContractError("expert id outside [0, E)")
    groups = [np.array([p for p in range(ids.size) if ids[p] == e], dtype=np.int64)
              for e in range(num_experts)]
    counts = np.array([g.size for g in groups], dtype=np.int64)
    return counts, groups


def collapse_w13_scale2(scale2: np.ndarray) -> tuple[np.ndarray, bool]:
    """E6: per-expert global scale of w13 (its w1 column) and whether w3's differs."""
    s = np.asarray(scale2, dtype=np.float32).reshape(scale2.shape[0], -1)
    return s[:, 0].copy(), bool(s.shape[1] > 1 and not np.array_equal(s[:, 0], s[:, 1]))


def grouped_gemm_ref(x_bits: np.ndarray, row_div: int, topk_ids: np.ndarray, packed: np.ndarray,
                     scales: np.ndarray, gs: np.ndarray):
    """E2 in fp64: ``(y64, w_norm, abs_sum)`` for every pair row.

    ``packed`` [E, N, K/2], ``scales`` [E, N, K/16], ``gs`` [E].  Returns the
    fp64 outputs [P, N], the 2-norm of the dequantized weight row each output
    uses [P, N], and ``sum_k |x| |w_deq|`` [P, N] (the magnitude that bounds
    float32 summation error).
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    E, N = packed.shape[0], packed.shape[1]
    _, groups = route(ids, E)
    x = O.bf16_bits_to_f32(x_bits).astype(np.float64)
    P = ids.size
    y = np.zeros((P, N))
    wn = np.zeros((P, N))
    sa = np.zeros((P, N))
    for e in range(E):
        rows = groups[e]
        if rows.size == 0:
            continue
        wd = O.dequantize(packed[e], scales[e], float(gs[e]))
        xe = x[rows // row_div]
        y[rows] = xe @ wd.T
        sa[rows] = np.abs(xe) @ np.abs(wd).T
        wn[rows] = np.linalg.norm(wd, axis=1)[None, :]
    return y, wn, sa


def gemm_bound(x_bits: np.ndarray, row_div: int, y64: np.ndarray, w_norm: np.ndarray,
               abs_sum: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-element bounds of one expert GEMM's bf16 output: (norm bound, tight bound).

    Norm bound: ``1e-3 * ||x_row||_2 * ||w_deq_n||_2`` plus half a bf16 ulp of
    the exact result.  Tight: float32 accumulation of exact products,
    ``(K + 2) * 2^-24 * sum|x w|``, plus one bf16 rounding, ``2^-8 |y|``.
    """
    x = O.bf16_bits_to_f32(x_bits).astype(np.float64)
    xn = np.linalg.norm(x, axis=1)
    P = y64.shape[0]
    xrow = xn[np.arange(P) // row_div]
    loose = 1e-3 * xrow[:, None] * w_norm + 2.0 ** -9 * np.abs(y64)
    tight = (K + 2) * 2.0 ** -24 * abs_sum + 2.0 ** -8 * np.abs(y64)
    return loose, tight


def silu(g: np.ndarray) -> np.ndarray:
    """E3 in fp64, without overflow for large negative g."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    eg = np.exp(g[~pos])
    out[~pos] = g[~pos] * eg / (1.0 + eg)
    return out


def silu_and_mul_ref(h_bits: np.ndarray) -> np.ndarray:
    """E3: bf16 ``h`` [P, 2I] -> fp64 ``silu(h[:, :I]) * h[:, I:]``."""
    h = O.bf16_bits_to_f32(h_bits).astype(np.float64)
    i = h.shape[1] // 2
    return silu(h[:, :i]) * h[:, i:]


def combine_ref(o_bits: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """E4: bf16 ``o`` [T * topk, H] and float32 weights [T, topk] -> fp64 [T, H]."""
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k = w.shape
    o = O.bf16_bits_to_f32(o_bits).astype(np.float64).reshape(T, k, -1)
    return np.einsum("tj,tjh->th", w, o)


def moe_ref(x_bits, topk_ids, topk_weights, w13, w2):
    """The whole layer in fp64 with no intermediate rounding, plus what its
    error bound needs.  ``w13`` / ``w2`` = (packed, scales, gs) per E2.

    Returns a dict: ``out`` [T, H], ``h`` [P, 2I], ``a`` [P, I], ``o`` [P, H],
    ``h_abs`` (``sum |x w|`` of the first GEMM), the dequantized w2 of each
    expert with pairs (``w2deq``) and the pairs of each expert (``groups``).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    h, _, h_abs = grouped_gemm_ref(x_bits, k, ids, *w13)
    i = h.shape[1] // 2
    a = silu(h[:, :i]) * h[:, i:]
    E = w2[0].shape[0]
    _, groups = route(ids, E)
    P = ids.size
    H = w2[0].shape[1]
    o = np.zeros((P, H))
    w2deq = [None] * E
    for e in range(E):
        if groups[e].size:
            w2deq[e] = O.dequantize(w2[0][e], w2[1][e], float(w2[2][e]))
            o[groups[e]] = a[groups[e]] @ w2deq[e].T
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    out = np.einsum("tj,tjh->th", w, o.reshape(T, k, H))
    return {"out": out, "h": h, "a": a, "o": o, "h_abs": h_abs, "w2deq": w2deq, "groups": groups}


def moe_tolerance(ref: dict, topk_weights: np.ndarray, K1: int) -> np.ndarray:
    """E5: first-order bound on |out_gpu - out64| per element.

    Each stage's error: the GEMM1 output ``dh = (K1+2) 2^-24 sum|x w| +
    2^-8 |h|`` (twice that, for the second-order term); the activation
    ``da = |silu'(g)| |u| dg + |silu(g)| du + dg du + 2^-8 |a| + 2^-20 |a|``
    (float32 evaluation); the second GEMM carries ``da`` through ``|w2|``, adds
    its own float32 sum over I terms and one bf16 rounding of ``o``; the
    combine adds float32 sums and one bf16 rounding of ``out``.
    """
    h, a, o, groups, w2deq = ref["h"], ref["a"], ref["o"], ref["groups"], ref["w2deq"]
    i = h.shape[1] // 2
    g, u = h[:, :i], h[:, i:]
    dh = 2.0 * ((K1 + 2) * 2.0 ** -24 * ref["h_abs"] + 2.0 ** -8 * np.abs(h))
    dg, du = dh[:, :i], dh[:, i:]
    sg = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    dsilu = np.abs(sg * (1.0 + g * (1.0 - sg))) + 0.1 * dg     # |silu'| <= 1.1 near the slope's peak
    da = dsilu * np.abs(u) * dg + np.abs(silu(g)) * du + dg * du + (2.0 ** -8 + 2.0 ** -20) * np.abs(a)
    P, H = o.shape
    do = np.zeros((P, H))
    for e, rows in enumerate(groups):
        if rows.size:
            wa = np.abs(w2deq[e])
            do[rows] = (da[rows] + np.abs(a[rows])) @ wa.T * 1.0   # |a| + da bounds the bf16 operand
            do[rows] = (da[rows] @ wa.T + (i + 2) * 2.0 ** -24 * do[rows]
                        + 2.0 ** -8 * np.abs(o[rows]) * (1 + 2.0 ** -7))
    w = np.abs(np.asarray(topk_weights, dtype=np.float32).astype(np.float64))
    T, k = w.shape
    dout = np.einsum("tj,tjh->th", w, do.reshape(T, k, H))
    out = ref["out"]
    oabs = np.einsum("tj,tjh->th", w, (np.abs(o) + do).reshape(T, k, H))
    return dout + (k + 2) * 2.0 ** -24 * oabs + 2.0 ** -8 * (np.abs(out) + dout)
