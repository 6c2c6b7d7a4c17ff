"""Host checks of arithmetic identities the GPU kernels rely on (no GPU, no oracle).

The block-scale rule needs fl32(b / 6) for the block max b (a non-negative
finite bf16).  The quantization kernel computes it without a division:
q0 = fl(b * fl(1/6)); r = fl(fma(-q0, 6, b)); q = fl(fma(r, fl(1/6), q0)).
This test evaluates that sequence exactly (each fma rounded once) for all
32 640 non-negative finite bf16 values and compares it with the correctly
rounded quotient.
"""

from fractions import Fraction

import numpy as np


def round_f32(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormals share the minimum exponent
    ulp = Fraction(2) ** (e - 23)
    q, rem = divmod(a, ulp)
    q = int(q)
    if rem * 2 > ulp or (rem * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(1)
    for x in rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000):
        assert float(round_f32(Fraction(float(x)))) == float(np.float32(x))


def test_div6_sequence_is_correctly_rounded_for_all_bf16():
    inv6 = Fraction(float(np.float32(1.0) / np.float32(6.0)))
    six = Fraction(6)
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16      # +0 .. largest finite bf16
    values = bits.view(np.float32)
    bad = []
    for b in values:
        fb = Fraction(float(b))
        q0 = round_f32(fb * inv6)
        r = round_f32(-q0 * six + fb)
        q = round_f32(r * inv6 + q0)
        if q != round_f32(fb / six):
            bad.append(float(b))
    assert not bad, f"{len(bad)} bf16 values differ, e.g. {bad[:5]}"
