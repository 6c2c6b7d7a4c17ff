"""Pins of the mixture-of-experts oracle (oracle/nvfp4_moe_oracle.py) against
library routines, closed forms and brute force (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle.nvfp4_oracle as O
import oracle.nvfp4_moe_oracle as MO
from nvfp4_w4a16_lm_amd import workloads as wl


def _experts(E, N, K, seed):
    bits = wl.moe_expert_bits(N, K, E, 0.02, 90 + seed, 0)
    qs = [O.quantize(bits[e]) for e in range(E)]
    packed = np.stack([q[0] for q in qs])
    scales = np.stack([q[1] for q in qs])
    gs = np.array([q[2] for q in qs], dtype=np.float32)
    return packed, scales, gs


def test_route_matches_stable_argsort_and_bincount():
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 7, size=200).astype(np.int32)
    counts, groups = MO.route(ids, 9)
    assert np.array_equal(counts, np.bincount(ids, minlength=9))
    assert np.array_equal(np.concatenate(groups), np.argsort(ids, kind="stable"))
    assert counts[7] == 0 and counts[8] == 0


def test_route_rejects_ids_outside_range():
    with pytest.raises(O.OracleContractError):
        MO.route(np.array([0, 3], np.int32), 3)
    with pytest.raises(O.OracleContractError):
        MO.route(np.array([-1], np.int32), 3)


def test_single_expert_equals_lm_head_gemm():
    packed, scales, gs = _experts(1, 48, 64, 0)
    x = wl.random_activation_bits(3, 64, seed=1)
    ids = np.zeros((3, 2), np.int32)
    y, wn, sa = MO.grouped_gemm_ref(x, 2, ids, packed, scales, gs)
    ref = O.gemm_ref(x, packed[0], scales[0], gs[0])
    assert np.array_equal(y, np.repeat(ref, 2, axis=0))
    assert np.allclose(wn[0], np.linalg.norm(O.dequantize(packed[0], scales[0], gs[0]), axis=1))


def test_one_hot_rows_give_dequantized_weights():
    E, N, K = 3, 32, 48
    packed, scales, gs = _experts(E, N, K, 1)
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80                  # bf16 1.0
    ids = (np.arange(K) % E).astype(np.int32)
    y, _, _ = MO.grouped_gemm_ref(x, 1, ids, packed, scales, gs)
    for p in range(K):
        e = ids[p]
        codes = O.unpack_codes(packed[e])[:, p]
        want = O.e2m1_value(codes) * O.e4m3_value(scales[e][:, p // 16]) * float(gs[e])
        assert np.array_equal(y[p], want)


def test_expert_relabelling_does_not_change_outputs():
    E, N, K = 4, 32, 64
    packed, scales, gs = _experts(E, N, K, 2)
    x = wl.random_activation_bits(6, K, seed=2)
    ids = np.array([[0, 3], [1, 2], [3, 1], [2, 0], [0, 1], [3, 2]], np.int32)
    y, _, _ = MO.grouped_gemm_ref(x, 2, ids, packed, scales, gs)
    perm = np.array([2, 0, 3, 1])                            # new label of old expert e
    inv = np.argsort(perm)
    y2, _, _ = MO.grouped_gemm_ref(x, 2, perm[ids].astype(np.int32), packed[inv], scales[inv], gs[inv])
    assert np.array_equal(y, y2)


def test_silu_against_library_logistic():
    g = np.concatenate([np.linspace(-30, 30, 2001), [-1000.0, -80.0, 0.0, 80.0, 1000.0]])
    assert np.allclose(MO.silu(g), g * scipy.special.expit(g), rtol=1e-15, atol=1e-300)
    assert MO.silu(np.array([0.0]))[0] == 0.0
    assert MO.silu(np.array([1000.0]))[0] == 1000.0
    assert abs(MO.silu(np.array([-1000.0]))[0]) < 1e-300


def test_silu_and_mul_gates_with_the_first_half():
    g = np.array([[1.0, -2.0, 3.0, 0.5]], np.float32)        # h = [g0 g1 | u0 u1]
    h = wl.f32_to_bf16_bits(g)
    a = MO.silu_and_mul_ref(h)
    assert np.allclose(a[0], [1.0 / (1 + np.exp(-1.0)) * 3.0, -2.0 / (1 + np.exp(2.0)) * 0.5], rtol=1e-15)
    swapped = MO.silu(np.array([3.0, 0.5])) * np.array([1.0, -2.0])
    assert not np.allclose(a[0], swapped)


def test_combine_exact_rationals():
    rng = np.random.default_rng(4)
    T, k, H = 3, 3, 8
    o = wl.f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    w = rng.uniform(0.1, 1, (T, k)).astype(np.float32)
    got = MO.combine_ref(o, w)
    of = O.bf16_bits_to_f32(o)
    for t in range(T):
        for h in range(H):
            exact = sum(Fraction(float(w[t, j])) * Fraction(float(of[t * k + j, h])) for j in range(k))
            assert abs(Fraction(got[t, h]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_combine_single_slot_unit_weight_is_identity():
    o = wl.random_activation_bits(4, 16, seed=5)
    got = MO.combine_ref(o, np.ones((4, 1), np.float32))
    assert np.array_equal(got, O.bf16_bits_to_f32(o).astype(np.float64))


def test_collapse_w13_scale2_keeps_w1_column():
    s = np.array([[0.5, 0.5], [0.25, 0.25]], np.float32)
    v, differ = MO.collapse_w13_scale2(s)
    assert np.array_equal(v, [0.5, 0.25]) and not differ
    v, differ = MO.collapse_w13_scale2(np.array([[0.5, 0.75]], np.float32))
    assert v[0] == np.float32(0.5) and differ


def test_moe_ref_equals_brute_force_loops():
    E, H, I, T, k = 3, 32, 16, 2, 2
    w13 = _experts(E, 2 * I, H, 3)
    w2 = _experts(E, H, I, 4)
    x = wl.random_activation_bits(T, H, seed=6)
    ids = np.array([[2, 0], [1, 2]], np.int32)
    tw = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    ref = MO.moe_ref(x, ids, tw, w13, w2)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = ids[t, j]
            W1 = O.dequantize(w13[0][e], w13[1][e], w13[2][e])
            W2 = O.dequantize(w2[0][e], w2[1][e], w2[2][e])
            h = np.array([sum(xf[t, kk] * W1[n, kk] for kk in range(H)) for n in range(2 * I)])
            a = h[:I] / (1 + np.exp(-h[:I])) * h[I:]
            o = np.array([sum(a[i] * W2[n, i] for i in range(I)) for n in range(H)])
            acc += float(tw[t, j]) * o
        assert np.allclose(ref["out"][t], acc, rtol=1e-12, atol=1e-300)


def test_tolerance_covers_the_bf16_rounding_chain():
    """Rounding every intermediate of the oracle's own fp64 chain to bf16 (what
    the GPU stores) stays within the bound, and the bound is not vacuous."""
    E, H, I, T, k = 4, 64, 32, 6, 2
    w13 = _experts(E, 2 * I, H, 5)
    w2 = _experts(E, H, I, 6)
    x = wl.random_activation_bits(T, H, seed=7)
    ids, tw = wl.moe_routing(T, E, k, 99)
    ref = MO.moe_ref(x, ids, tw, w13, w2)
    tol = MO.moe_tolerance(ref, tw, H)
    r16 = lambda v: O.bf16_round_rne(v)                        # noqa: E731
    h = r16(ref["h"])
    a = r16(MO.silu(h[:, :I]) * h[:, I:])
    o = np.zeros_like(ref["o"])
    for e, rows in enumerate(ref["groups"]):
        if rows.size:
            o[rows] = r16(a[rows] @ O.dequantize(w2[0][e], w2[1][e], w2[2][e]).T)
    out = r16(np.einsum("tj,tjh->th", tw.astype(np.float64), o.reshape(T, k, H)))
    assert np.all(np.abs(out - ref["out"]) <= tol)
    # not vacuous: plausible mistakes leave it on most elements
    h_sw = np.concatenate([ref["h"][:, I:], ref["h"][:, :I]], axis=1)     # gate and up swapped
    a_sw = MO.silu(h_sw[:, :I]) * h_sw[:, I:]
    o_sw = np.zeros_like(ref["o"])
    for e, rows in enumerate(ref["groups"]):
        if rows.size:
            o_sw[rows] = a_sw[rows] @ O.dequantize(w2[0][e], w2[1][e], w2[2][e]).T
    out_sw = np.einsum("tj,tjh->th", tw.astype(np.float64), o_sw.reshape(T, k, H))
    assert np.mean(np.abs(out_sw - ref["out"]) > tol) > 0.5   # small h: silu(g) u ~ g u / 2 is nearly symmetric
    out_nw = ref["o"].reshape(T, k, H).sum(axis=1)                          # routing weights dropped
    assert np.mean(np.abs(out_nw - ref["out"]) > tol) > 0.9
