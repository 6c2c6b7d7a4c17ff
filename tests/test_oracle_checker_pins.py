"""Pins for the oracle functions every GPU GEMM check relies on.

``gemm_ref_with_norms`` gives the fp64 logits, the weight-row 2-norms and the
sums ``sum_k |x| |w_deq|`` that the norm bound and the tight bound are built
from; ``gemm_tolerance`` is the smoke check's norm bound; ``bf16_round_rne``
is the expected value of the one-hot GPU test.  (Vocabulary and bound: vLLM
API docs, quantization.online.lm_head, _LMHeadNvfp4Method.apply computes the
logits x . W_deq^T with activations in the model dtype; the tolerance is the
per-element 1e-3 ||x_m|| ||w_n|| bound.)

Each function is checked against something other than itself: exact rational
arithmetic over dequantized values built from the format definitions
(not the oracle's dequantizer), hand-computed closed forms, and torch's
float32 -> bfloat16 cast.  The last section plants plausible mistakes (a
dropped ``abs``, a norm over the wrong axis, a lost bias, truncation instead
of rounding) in a copy of the oracle and checks that the pins catch each.
"""

import math
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import workloads as wl

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_fraction(byte: int) -> Fraction:
    """Value of a non-negative float8_e4m3fn byte (1-4-3, bias 7, subnormal step 2^-9)."""
    e, m = byte >> 3, byte & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def deq_fractions(packed, scales, gs):
    """Dequantized weights as exact rationals, from the code table and the E4M3
    definition: code nibbles low first, bit 3 the sign."""
    n, h = packed.shape
    out = []
    for r in range(n):
        row = []
        for i in range(h):
            for c in (int(packed[r, i]) & 0xF, int(packed[r, i]) >> 4):
                k = len(row)
                v = GRID[c & 7] * e4m3_fraction(int(scales[r, k // 16])) * Fraction(float(gs))
                row.append(-v if c & 8 else v)
        out.append(row)
    return out


def small_case(n=5, k=48, m=3, seed=7, bias=True):
    w = wl.random_weight_bits(n, k, sigma=0.3, seed=seed)
    x = wl.random_activation_bits(m, k, seed=seed)
    b = wl.bias_bits(n, seed=seed) if bias else None
    packed, scales, gs = O.quantize(w)
    return x, packed, scales, gs, b


# ---------------------------------------------------------------------------
# checks, each taking the module under test
# ---------------------------------------------------------------------------

def check_y_matches_gemm_ref(o):
    """The logits of gemm_ref_with_norms are gemm_ref's, bit for bit, with and
    without bias, also when the rows are walked in several chunks."""
    for bias in (False, True):
        x, packed, scales, gs, b = small_case(n=7, k=64, m=4, seed=11, bias=bias)
        for chunk in (8192, 3):
            y, _, _ = o.gemm_ref_with_norms(x, packed, scales, gs, b, chunk_rows=chunk)
            assert np.array_equal(y, o.gemm_ref(x, packed, scales, gs, b)), (bias, chunk)


def check_y_exact_rational(o):
    """y64 equals the exact rational sum within fp64 rounding of K products."""
    x, packed, scales, gs, b = small_case(n=4, k=32, m=2, seed=3)
    y, _, _ = o.gemm_ref_with_norms(x, packed, scales, gs, b)
    wd = deq_fractions(packed, scales, gs)
    xf = wl.bf16_bits_to_f32(x)
    bf = wl.bf16_bits_to_f32(b)
    for mi in range(2):
        for n in range(4):
            acc = sum(Fraction(float(xf[mi, kk])) * wd[n][kk] for kk in range(32)) + Fraction(float(bf[n]))
            mag = sum(abs(Fraction(float(xf[mi, kk])) * wd[n][kk]) for kk in range(32)) + abs(Fraction(float(bf[n])))
            assert abs(Fraction(float(y[mi, n])) - acc) <= mag * Fraction(40, 2 ** 53)


def check_row_norms(o):
    """w_norm[n] is the 2-norm of dequantized row n: its square equals the exact
    rational sum of squares within a few fp64 roundings.  A square shape
    (N == K) makes a norm over the wrong axis give wrong values, not an error."""
    for n, k in ((6, 48), (32, 32)):
        w = wl.random_weight_bits(n, k, sigma=0.2, seed=n + k)
        packed, scales, gs = O.quantize(w)
        x = wl.random_activation_bits(2, k, seed=5)
        _, wn, _ = o.gemm_ref_with_norms(x, packed, scales, gs)
        assert wn.shape == (n,)
        wd = deq_fractions(packed, scales, gs)
        for r in range(n):
            sq = sum(v * v for v in wd[r])
            assert abs(Fraction(float(wn[r])) ** 2 - sq) <= sq * Fraction(4 * k + 8, 2 ** 53), r


def check_abs_sums(o):
    """s_abs[m, n] = sum_k |x[m,k]| |w_deq[n,k]| against exact rationals."""
    x, packed, scales, gs, b = small_case(n=5, k=48, m=3, seed=9)
    _, _, s_abs = o.gemm_ref_with_norms(x, packed, scales, gs, b)
    assert s_abs.shape == (3, 5)
    wd = deq_fractions(packed, scales, gs)
    xf = wl.bf16_bits_to_f32(x)
    for mi in range(3):
        for n in range(5):
            want = sum(abs(Fraction(float(xf[mi, kk]))) * abs(wd[n][kk]) for kk in range(48))
            assert abs(Fraction(float(s_abs[mi, n])) - want) <= want * Fraction(60, 2 ** 53), (mi, n)


def grid_weight():
    """Two rows of 32 weights whose quantization is known in closed form.

    With max|W| = 2688 = 6 * 448 the global scale is exactly 1.  Row 0 holds
    2688 at k = 0 and zeros: block 0 gets scale 448 (byte 0x7E) and code 7,
    block 1 is a zero block (scale 0).  Row 1 holds 2688 at k = 0 and 1344 at
    k = 16: block 1's scale is 1344 / 6 = 224 (exact in E4M3) and its code 7.
    Dequantized: row 0 = [2688, 0, ...], row 1 = [2688, 0 x 15, 1344, 0 x 15]."""
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, 0] = 2688.0
    w[1, 0] = 2688.0
    w[1, 16] = 1344.0
    return wl.f32_to_bf16_bits(w)


def check_tolerance_closed_form(o):
    """gemm_tolerance = 1e-3 ||x_m|| ||w_n|| (+ 2^-8 |bias_n|), hand-computed."""
    packed, scales, gs = O.quantize(grid_weight())
    assert float(gs) == 1.0 and int(scales[0, 0]) == 0x7E and int(scales[1, 1]) == 0x76
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0          # ||x_0|| = 5
    x[1, :] = 1.0                        # ||x_1|| = sqrt(32)
    xb = wl.f32_to_bf16_bits(x)
    w0, w1 = 2688.0, 1344.0 * math.sqrt(5.0)          # ||w_0||, ||w_1||
    want = 1e-3 * np.array([[5.0 * w0, 5.0 * w1], [math.sqrt(32) * w0, math.sqrt(32) * w1]])
    got = o.gemm_tolerance(xb, packed, scales, gs)
    assert got.shape == (2, 2)
    assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)
    bias = wl.f32_to_bf16_bits(np.array([2.0, -0.5], dtype=np.float32))
    got_b = o.gemm_tolerance(xb, packed, scales, gs, bias_bits=bias)
    assert np.allclose(got_b, want + np.array([[2.0 ** -7, 2.0 ** -9]]), rtol=1e-12, atol=0), got_b
    # rtol scales the norm part only
    got_r = o.gemm_tolerance(xb, packed, scales, gs, rtol=1e-2, bias_bits=bias)
    assert np.allclose(got_r, 10 * want + np.array([[2.0 ** -7, 2.0 ** -9]]), rtol=1e-12, atol=0)


def check_norms_closed_form(o):
    """gemm_ref_with_norms on the closed-form weights: norms 2688 and 1344 sqrt(5),
    logits and |x||w| sums by hand."""
    packed, scales, gs = O.quantize(grid_weight())
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 16] = -0.5, 0.25
    y, wn, s_abs = o.gemm_ref_with_norms(wl.f32_to_bf16_bits(x), packed, scales, gs)
    assert np.allclose(wn, [2688.0, 1344.0 * math.sqrt(5.0)], rtol=1e-15, atol=0)
    assert np.array_equal(y, [[-1344.0, -1344.0 + 336.0]])
    assert np.array_equal(s_abs, [[1344.0, 1344.0 + 336.0]])


def bf16_inputs():
    rng = np.random.default_rng(12)
    rand = (rng.standard_normal(4000) * np.exp2(rng.integers(-140, 120, 4000))).astype(np.float32)
    # exact ties: the low 16 bits are 0x8000, with even and odd kept halves
    hi = rng.integers(0, 0x7F7F, 2000).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    near = np.concatenate([((hi << 16) | d).view(np.float32) for d in (0x7FFF, 0x8001, 0x0001, 0xFFFF)])
    # float32 subnormals (and their ties) and small normals
    sub = np.concatenate([np.arange(1, 200, dtype=np.uint32), np.uint32(0x8000) + np.arange(0, 200, dtype=np.uint32),
                          np.uint32(0x007F8000) + np.arange(0, 4, dtype=np.uint32),
                          np.uint32(0x00800000) + np.arange(0, 300, dtype=np.uint32) * np.uint32(0x4000)])
    sub = sub.view(np.float32)
    vals = np.concatenate([rand, ties, near, sub, np.float32([0.0, 1.0, 3.0, 1.00390625, 1.01171875])])
    return np.concatenate([vals, -vals]).astype(np.float32)


def check_bf16_round_rne(o):
    """bf16_round_rne equals torch's float32 -> bfloat16 cast (round to nearest
    even) on random, tie, near-tie and subnormal values, both signs."""
    f = bf16_inputs()
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = o.bf16_round_rne(f.astype(np.float64))
    assert got.dtype == np.float64
    same = (got == want) & (np.signbit(got) == np.signbit(want))
    assert np.all(same), f"first mismatch at {f[~same][0]!r}: {got[~same][0]!r} vs {want[~same][0]!r}"


CHECKS = [check_y_matches_gemm_ref, check_y_exact_rational, check_row_norms, check_abs_sums,
          check_tolerance_closed_form, check_norms_closed_form, check_bf16_round_rne]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_checker_pin(check):
    check(O)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one check above
# ---------------------------------------------------------------------------

def mutant(**overrides):
    m = types.ModuleType("oracle_checker_mutant")
    m.__dict__.update({k: v for k, v in vars(O).items() if not k.startswith("__")})
    m.__dict__.update(overrides)
    for name, obj in list(m.__dict__.items()):
        if isinstance(obj, types.FunctionType) and name not in overrides:
            m.__dict__[name] = types.FunctionType(obj.__code__, m.__dict__, name, obj.__defaults__, obj.__closure__)
    return m


def _norms_variant(no_abs=False, wrong_axis=False, drop_bias=False, no_gs=False):
    def fn(x_bits, packed, scales, gs, bias_bits=None, chunk_rows=8192):
        x = O.bf16_bits_to_f32(x_bits).astype(np.float64)
        xa = x if no_abs else np.abs(x)
        wd = O.dequantize(packed, scales, 1.0 if no_gs else gs)
        y = x @ wd.T
        s_abs = xa @ (wd if no_abs else np.abs(wd)).T
        wn = np.linalg.norm(wd, axis=0 if wrong_axis else 1)
        if bias_bits is not None and not drop_bias:
            y = y + O.bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
        return y, wn, s_abs
    return fn


def _tolerance_variant(wrong_axis=False, drop_bias=False, x_norm_sq=False):
    def fn(x_bits, packed, scales, gs, rtol=1e-3, bias_bits=None, chunk_rows=8192):
        x = O.bf16_bits_to_f32(x_bits).astype(np.float64)
        xn = np.sum(x * x, axis=1) if x_norm_sq else np.linalg.norm(x, axis=1)
        wd = O.dequantize(packed, scales, gs)
        wn = np.linalg.norm(wd, axis=0 if wrong_axis else 1)
        tol = rtol * xn[:, None] * wn[None, :]
        if bias_bits is not None and not drop_bias:
            tol = tol + 2.0 ** -8 * np.abs(O.bf16_bits_to_f32(bias_bits).astype(np.float64))[None, :]
        return tol
    return fn


def _bf16_truncate(y):
    bits = np.asarray(y, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return bits.view(np.float32).astype(np.float64)


def _bf16_ties_away(y):
    bits = np.asarray(y, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((bits + np.uint64(0x8000)) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _failures(o):
    failed = 0
    for c in CHECKS:
        try:
            c(o)
        except Exception:
            failed += 1
    return failed


@pytest.mark.parametrize("name,overrides", [
    ("abs sums without abs", {"gemm_ref_with_norms": _norms_variant(no_abs=True)}),
    ("row norm over the wrong axis", {"gemm_ref_with_norms": _norms_variant(wrong_axis=True)}),
    ("logits lose the bias", {"gemm_ref_with_norms": _norms_variant(drop_bias=True)}),
    ("weights without the global scale", {"gemm_ref_with_norms": _norms_variant(no_gs=True)}),
    ("tolerance norm over the wrong axis", {"gemm_tolerance": _tolerance_variant(wrong_axis=True)}),
    ("tolerance loses the bias term", {"gemm_tolerance": _tolerance_variant(drop_bias=True)}),
    ("tolerance squares ||x||", {"gemm_tolerance": _tolerance_variant(x_norm_sq=True)}),
    ("bf16 truncation", {"bf16_round_rne": _bf16_truncate}),
    ("bf16 ties away from zero", {"bf16_round_rne": _bf16_ties_away}),
])
def test_checker_mistakes_are_caught(name, overrides):
    assert _failures(O) == 0
    assert _failures(mutant(**overrides)) >= 1, name
