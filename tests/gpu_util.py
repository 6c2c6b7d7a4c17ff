"""Helpers for the GPU parity tests (host <-> device marshalling, comparisons)."""

from __future__ import annotations

import concurrent.futures

import numpy as np
import torch

import oracle.fp8_oracle as F
import oracle.nvfp4_oracle as O
import oracle.nvfp4_w4a4_oracle as A
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def quantize_gpu(w_bits: np.ndarray):
    p, s, g = B.nvfp4_quantize(dev_bf16(w_bits))
    torch.cuda.synchronize()
    return p.cpu().numpy(), s.view(torch.uint8).cpu().numpy(), np.float32(g.cpu().item())


def upload_quant(packed: np.ndarray, scales: np.ndarray, gs) -> tuple:
    return (dev_u8(packed), dev_u8(scales),
            torch.tensor(np.float32(gs), dtype=torch.float32, device=DEV))


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def assert_quant_equal(w_bits, got, want, label=""):
    gp, gsb, ggs = got
    wp, wsb, wgs = want
    assert f32_bits(ggs) == f32_bits(wgs), f"{label}: global scale {ggs!r} != {wgs!r}"
    bad_s = np.argwhere(gsb != wsb)
    bad_p = np.argwhere(gp != wp)
    if len(bad_s) or len(bad_p):
        n, j = (bad_s[0] if len(bad_s) else (bad_p[0][0], bad_p[0][1] // 8))
        blk = w_bits[n, 16 * j:16 * j + 16]
        raise AssertionError(
            f"{label}: {len(bad_s)} scale and {len(bad_p)} packed mismatches; first at row {n} block {j}: "
            f"scale gpu={gsb[n, j]:#04x} oracle={wsb[n, j]:#04x}; packed gpu={gp[n, 8*j:8*j+8].tolist()} "
            f"oracle={wp[n, 8*j:8*j+8].tolist()}; weights={wl.bf16_bits_to_f32(blk).tolist()}")


def oracle_quantize_threaded(w_bits: np.ndarray, gs, rows: int = 2048):
    """Oracle quantize_rows over row chunks on a thread pool (same arithmetic)."""
    n, k = w_bits.shape
    packed = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, k // 16), np.uint8)

    def work(r0):
        p, s = O.quantize_rows(w_bits[r0:r0 + rows], gs)
        packed[r0:r0 + rows] = p
        scales[r0:r0 + rows] = s

    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        list(ex.map(work, range(0, n, rows)))
    return packed, scales


def gemm_gpu(x_bits, qdev, bias_bits=None):
    p, s, g = qdev
    bias = None if bias_bits is None else dev_bf16(bias_bits)
    y = B.nvfp4_w4a16_gemm(dev_bf16(x_bits), p, s, g, bias)
    torch.cuda.synchronize()
    return host_bits(y)


def half_ulp_bf16(v):
    """Half a bf16 unit in the last place at |v| (0 for v == 0)."""
    _, ex = np.frexp(np.abs(v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 9))


def check_gemm(y_bits, x_bits, packed, scales, gs, bias_bits=None, label="", argmax_min=0.999,
               pure_bound=None):
    """Norm bound, tight fp32/bf16 bound and tie-aware argmax against the oracle.

    The norm bound 1e-3 * ||x_m|| * ||w_n|| is applied to the bf16 output,
    so half a bf16 ulp of the exact logit (the rounding any bf16 result carries)
    is added to it.  With ``pure_bound`` (default: K >= 512, where |cos(x_m, w_n)|
    stays far below 0.25 for these inputs) the bound must also hold without it.
    """
    y = wl.bf16_bits_to_f32(y_bits).astype(np.float64)
    y64, wn, s_abs = O.gemm_ref_with_norms(x_bits, packed, scales, gs, bias_bits)
    xn = np.linalg.norm(wl.bf16_bits_to_f32(x_bits).astype(np.float64), axis=1)
    bias_abs = 0.0 if bias_bits is None else np.abs(wl.bf16_bits_to_f32(bias_bits).astype(np.float64))[None, :]
    # norm bound: 1e-3 * ||x_m|| * ||w_n|| (+ bf16 rounding of a bias term)
    tol = 1e-3 * xn[:, None] * wn[None, :] + 2.0 ** -8 * bias_abs
    err = np.abs(y - y64)
    if pure_bound is None:
        pure_bound = x_bits.shape[1] >= 512
    if pure_bound:
        worst = np.unravel_index(np.argmax(err - tol), err.shape)
        assert np.all(err <= tol), (f"{label}: norm bound (no output-rounding term) broken at "
                                    f"{worst}: y={y[worst]} y64={y64[worst]} tol={tol[worst]}")
    tol = tol + half_ulp_bf16(y64)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"{label}: norm bound broken at {worst}: y={y[worst]} "
                                f"y64={y64[worst]} tol={tol[worst]}")
    # tight bound: fp32 accumulation of K exact products in any order, the scale and
    # bias operations, then one round-to-nearest to bf16.  The f16 decode route
    # stores each activation row as x * 2^-p with max |x * 2^-p| in [2^14, 2^15):
    # an activation may then move by at most max(2^-39 max|x_m|, 2^-151) (f16
    # subnormal spacing), i.e. by at most that times sum_k |w_k| <= sqrt(K) ||w_n||.
    k = x_bits.shape[1]
    xmax = np.max(np.abs(wl.bf16_bits_to_f32(x_bits).astype(np.float64)), axis=1)
    conv = (2.0 ** -39 * xmax + 2.0 ** -151)[:, None] * np.sqrt(k) * wn[None, :]
    acc = (k + 2) * 2.0 ** -24 * (s_abs + bias_abs) + conv
    tight = 1.01 * (acc + 2.0 ** -8 * (np.abs(y64) + acc)) + 2.0 ** -133
    worst = np.unravel_index(np.argmax(err - tight), err.shape)
    assert np.all(err <= tight), (f"{label}: tight bound broken at {worst}: y={y[worst]} "
                                  f"y64={y64[worst]} tight={tight[worst]}")
    if y.shape[1] > 1:
        tie, strict = O.argmax_agreement(y, y64)
        assert tie >= argmax_min, f"{label}: tie-aware argmax agreement {tie} (strict {strict})"
    return y64


def check_fp8_gemm(y_bits, xq, xs, wq, ws, bias_bits=None, label="", argmax_min=0.999):
    """Norm bound 1e-3 |x_m| |w_n| on the dequantized operands, and a
    tight bound for the arithmetic: v_mfma_f32_16x16x32_fp8_fp8 sums its 32
    products in reduced precision (errors up to 2^-16.7 of sum|x w| were
    measured on single instructions, far more than float32 rounding), so the
    bound allows 2^-14 sum|x w| s_x s_w for the instructions plus float32
    accumulation across them and the final bf16 rounding."""
    y = wl.bf16_bits_to_f32(y_bits).astype(np.float64)
    y64 = F.gemm_ref(xq, xs, wq, ws, bias_bits)
    yabs = F.gemm_abs_ref(xq, xs, wq, ws, bias_bits)
    xn = np.linalg.norm(F.e4m3_decode_signed(xq) * np.asarray(xs, np.float64)[:, None], axis=1)
    wn = np.linalg.norm(F.e4m3_decode_signed(wq) * np.asarray(ws, np.float64)[:, None], axis=1)
    ns = 1e-3 * xn[:, None] * wn[None, :] + 2.0 ** -8 * np.abs(y64)
    assert np.all(np.abs(y - y64) <= ns), f"{label}: norm bound"
    k = xq.shape[1]
    acc = (2.0 ** -14 + (k + 4) * 2.0 ** -24) * yabs
    tight = 1.01 * (acc + 2.0 ** -8 * (np.abs(y64) + acc)) + 2.0 ** -133
    err = np.abs(y - y64)
    worst = np.unravel_index(np.argmax(err - tight), err.shape)
    assert np.all(err <= tight), (f"{label}: |err| {err[worst]:.3e} > bound {tight[worst]:.3e} at {worst}: "
                                  f"gpu {y[worst]!r} ref {y64[worst]!r}")
    if argmax_min > 0 and y.shape[1] > 1:
        # tie-aware: the reference winner's bf16 logit equals the row's bf16 maximum
        win = np.argmax(y64, axis=1)
        ok = y[np.arange(y.shape[0]), win] == y.max(axis=1)
        assert ok.mean() >= argmax_min, f"{label}: argmax agreement {ok.mean():.4f}"


def check_w4a4(y_bits, xp, xs, wp, ws, a, bias_bits=None, label="", argmax_min=0.999):
    y = wl.bf16_bits_to_f32(y_bits).astype(np.float64)
    y64 = A.gemm_ref(xp, xs, wp, ws, a, bias_bits)
    yabs = A.gemm_abs_ref(xp, xs, wp, ws, a, bias_bits)
    xn = np.linalg.norm(A.block_values(xp, xs), axis=1)
    wn = np.linalg.norm(A.block_values(wp, ws), axis=1)
    ns = 1e-3 * float(a) * xn[:, None] * wn[None, :] + 2.0 ** -8 * np.abs(y64)
    err = np.abs(y - y64)
    assert np.all(err <= ns), f"{label}: norm bound"
    k = xp.shape[1] * 2
    acc = (k + 4) * 2.0 ** -24 * yabs
    tight = 1.01 * (acc + 2.0 ** -8 * (np.abs(y64) + acc)) + 2.0 ** -133
    worst = np.unravel_index(np.argmax(err - tight), err.shape)
    assert np.all(err <= tight), (f"{label}: |err| {err[worst]:.3e} > {tight[worst]:.3e} at {worst}: "
                                  f"gpu {y[worst]!r} ref {y64[worst]!r}")
    if argmax_min > 0 and y.shape[1] > 1:
        win = np.argmax(y64, axis=1)
        ok = y[np.arange(y.shape[0]), win] == y.max(axis=1)
        assert ok.mean() >= argmax_min, f"{label}: argmax agreement {ok.mean():.4f}"
