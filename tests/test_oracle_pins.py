"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these re-types the oracle's own formulas.  They use the values the
pages print (tests/golden/page_facts.json), a hand-derived worked example
(tests/golden/worked_example.json), brute-force nearest-value searches, exact
rational arithmetic, torch's float8_e4m3fn cast (the library cast the
quantizer on the vLLM API docs page applies to its block scales), closed forms
and invariants.  The last section plants plausible mistakes in a copy of the
oracle and checks that the pins catch each of them.
"""

import copy
import json
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import workloads as wl

F32 = np.float32


# ---------------------------------------------------------------------------
# independent helpers (brute force / exact arithmetic)
# ---------------------------------------------------------------------------

def e4m3_table():
    """All 127 finite non-negative float8_e4m3fn values by byte, from the format
    definition (1-4-3, bias 7, subnormal step 2^-9, 0x7F is NaN)."""
    vals = {}
    for byte in range(0x7F):
        e, m = byte >> 3, byte & 7
        vals[byte] = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return vals


E4M3 = e4m3_table()
E4M3_BYTES = np.array(sorted(E4M3), dtype=np.int64)
E4M3_VALUES = np.array([float(E4M3[b]) for b in sorted(E4M3)], dtype=np.float64)


def brute_e4m3(u):
    """Nearest e4m3 value by exhaustive search, ties to the even mantissa."""
    u = np.asarray(u, dtype=np.float64)
    d = np.abs(u[:, None] - E4M3_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates take the one whose byte (mantissa LSB) is even
    even = cand & ((E4M3_BYTES[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return E4M3_BYTES[pick].astype(np.uint8)


E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def brute_e2m1(a):
    """Nearest E2M1 magnitude by search over the 8 grid values, ties to the even code."""
    a = np.asarray(a, dtype=np.float64)
    d = np.abs(a[:, None] - E2M1_GRID[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(8)
    even = cand & ((codes[None, :] & 1) == 0)
    return np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)


def f32_round_fraction(fr):
    """Correctly rounded float32 of an exact rational (ties to even)."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))]
    best = min(abs(Fraction(float(x)) - fr) for x in cands)
    ties = [x for x in cands if abs(Fraction(float(x)) - fr) == best]
    if len(ties) > 1:
        ties = [x for x in ties if (np.array(x, dtype=np.float32).view(np.uint32) & 1) == 0]
    return ties[0]


def around(values, ulps=4):
    """Every float32 within ``ulps`` ulps of each value (non-negative only)."""
    out = []
    for v in values:
        x = F32(v)
        lo = hi = x
        out.append(x)
        for _ in range(ulps):
            lo = np.nextafter(lo, F32(-np.inf))
            hi = np.nextafter(hi, F32(np.inf))
            out.extend([lo, hi])
    out = np.array(out, dtype=np.float32)
    return out[out >= 0]


def bits_of(values):
    return wl.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# pin checks (take the oracle module so the mutation tests can reuse them)
# ---------------------------------------------------------------------------

def check_code_table(o, facts):
    t = facts["e2m1_code_table"]
    dm = np.array(t["doubled_magnitudes"], dtype=np.float64)
    codes = np.array(t["codes"], dtype=np.uint8)
    # decoding a code gives half its doubled magnitude
    assert np.array_equal(o.e2m1_value(codes), dm / 2)
    # encoding each grid magnitude gives its code
    assert np.array_equal(o.e2m1_magnitude_code((dm / 2).astype(np.float32)), codes)


def check_sign_and_zero(o, facts):
    bit = facts["sign_bit"]["bit"]
    for c in range(8):
        assert o.e2m1_value(np.array([c | (1 << bit)], np.uint8))[0] == -o.e2m1_value(np.array([c], np.uint8))[0]
    # -0.0 and values rounding to zero encode as code 0 (no sign); a whole-row check
    w = bits_of([1.0, -0.0, -1e-6, -0.02, -1.0] + [0.0] * 11)[None, :]
    packed, _, _ = o.quantize(w)
    codes = o.unpack_codes(packed)[0]
    assert codes[0] == 7 and codes[4] == 0xF
    assert codes[1] == 0 and codes[2] == 0 and codes[3] == 0


def check_packing(o, facts):
    p = facts["packing"]
    c = np.array([p["example_codes"]], dtype=np.uint8)
    assert o.pack_codes(c)[0, 0] == p["example_byte"]
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(3, 32), dtype=np.uint8)
    packed = o.pack_codes(codes)
    assert packed.shape == (3, 16)
    for i in range(16):
        assert np.array_equal(packed[:, i] & 0xF, codes[:, 2 * i])
        assert np.array_equal(packed[:, i] >> 4, codes[:, 2 * i + 1])


def check_worked_example(o, ex):
    w = np.array(ex["weights"], dtype=np.float64)
    for idx, val in ex["exact_weights"].items():
        if idx.startswith("_"):
            continue
        mant, e = val
        w[int(idx)] = mant * 2.0 ** e
    wb = bits_of(w.astype(np.float32))[None, :]
    # every weight must be exactly representable in bf16
    assert np.array_equal(wl.bf16_bits_to_f32(wb)[0].astype(np.float64), w)
    packed, scales, gs = o.quantize(wb)
    assert float(gs) == ex["expected_gs"]
    assert scales[0].tolist() == ex["expected_scales"]
    assert o.unpack_codes(packed)[0].tolist() == ex["expected_codes"]


def check_gs_exhaustive(o):
    """All 32640 non-negative finite bf16 amax values against exact rationals."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    clamp = f32_round_fraction(Fraction(1e-12))
    for a in amax:
        gs = o.global_scale(F32(a))
        want = f32_round_fraction(Fraction(float(a)) / 2688)
        want = max(want, clamp)
        assert np.float32(gs) == want, a
        inv = o.inverse_global_scale(gs)
        assert np.float32(inv) == f32_round_fraction(1 / Fraction(float(want)))


def check_gs_closed_forms(o):
    for k in range(-30, 30):
        a = F32(2688.0 * 2.0 ** k)
        gs = o.global_scale(a)
        if 2.0 ** k >= 1e-12:
            assert gs == F32(2.0 ** k)
            assert o.inverse_global_scale(gs) == F32(2.0 ** -k)
    assert np.float32(o.global_scale(F32(6.0))).view(np.uint32) == 0x3B124925
    assert o.inverse_global_scale(o.global_scale(F32(6.0))) == F32(447.99997)
    assert np.float32(o.global_scale(F32(0.0))).view(np.uint32) == np.float32(1e-12).view(np.uint32)


def e4m3_probe_inputs(n_random=200_000):
    vals = E4M3_VALUES
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(11)
    u = np.concatenate([
        around(vals), around(mids),
        rng.uniform(0, 448, n_random).astype(np.float32),
        np.exp2(rng.uniform(-14, np.log2(448), n_random)).astype(np.float32),
    ])
    return np.clip(u, 0, 448).astype(np.float32)


def check_e4m3_bruteforce(o):
    u = e4m3_probe_inputs()
    assert np.array_equal(o.e4m3_encode_rne(u), brute_e4m3(u))


def check_e4m3_decode(o):
    for byte, v in E4M3.items():
        assert o.e4m3_value(np.array([byte], np.uint8))[0] == float(v)


def e2m1_probe_inputs():
    grid = E2M1_GRID
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(12)
    a = np.concatenate([around(grid), around(mids), rng.uniform(0, 6, 200_000).astype(np.float32)])
    return np.clip(a, 0, 6).astype(np.float32)


def check_e2m1_bruteforce(o):
    a = e2m1_probe_inputs()
    assert np.array_equal(o.e2m1_magnitude_code(a), brute_e2m1(a))


def check_block_max_invariant(o, w_bits):
    packed, scales, gs = o.quantize(w_bits)
    codes = o.unpack_codes(packed)
    n, k = w_bits.shape
    w = np.abs(wl.bf16_bits_to_f32(w_bits)).reshape(n, k // 16, 16)
    arg = w.argmax(axis=2)
    s = o.e4m3_value(scales)
    mag = (codes.reshape(n, k // 16, 16) & 7)
    top = np.take_along_axis(mag, arg[:, :, None], axis=2)[:, :, 0]
    normal = s >= 2.0 ** -6
    assert normal.any()
    assert np.all(top[normal] == 7)


def check_dequant_error_bound(o, w_bits):
    """|w - deq(w)| <= (1/(1-1/16)) * b/6 (+ rounding) for blocks with normal scales."""
    packed, scales, gs = o.quantize(w_bits)
    n, k = w_bits.shape
    w = wl.bf16_bits_to_f32(w_bits).astype(np.float64)
    deq = o.dequantize(packed, scales, gs)
    err = np.abs(w - deq).reshape(n, k // 16, 16).max(axis=2)
    b = np.abs(w).reshape(n, k // 16, 16).max(axis=2)
    s = o.e4m3_value(scales)
    normal = s >= 2.0 ** -6
    bound = b / 6 * (16 / 15) * (1 + 1e-5)
    assert np.all(err[normal] <= bound[normal])
    # and the error is not trivially zero (the format is lossy)
    assert err.max() > 0


def check_grid_roundtrip(o):
    rng = np.random.default_rng(5)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    n, k = 8, 64
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    codes[:, ::16] = 7                     # +6 in every block
    codes[:, 5::16] = 0xF                  # and -6
    vals = np.where(codes & 8, -1.0, 1.0) * grid[codes & 7]
    want = np.where((codes & 7) == 0, 0, codes).astype(np.uint8)   # -0 encodes as 0
    # (i) any positive factor that keeps scales >= 2^-7: codes are preserved
    for f in [1.0, 0.37, 3.1e-3, 17.0, 1e4]:
        wb = bits_of(vals * np.float32(f))
        # bf16 rounding of the scaled grid must keep the ratios exact: use powers of 2 there
        if not np.array_equal(wl.bf16_bits_to_f32(wb).astype(np.float64), (vals * np.float32(f)).astype(np.float64)):
            continue
        packed, scales, gs = o.quantize(wb)
        assert np.all(o.e4m3_value(scales) >= 2.0 ** -7)
        assert np.array_equal(o.unpack_codes(packed), want)
    # (ii) scaled by 448 * 2^j: scales all 0x7E, gs = 2^j, exact dequantization
    for j in [-20, -3, 0, 5]:
        wb = bits_of(vals * np.float32(448.0 * 2.0 ** j))
        packed, scales, gs = o.quantize(wb)
        assert gs == F32(2.0 ** j)
        assert np.all(scales == 0x7E)
        assert np.array_equal(o.unpack_codes(packed), want)
        assert np.array_equal(o.dequantize(packed, scales, gs), wl.bf16_bits_to_f32(wb).astype(np.float64))
    # (iii) a block without +-6 is rescaled so its max maps to 6: codes change
    small = np.tile(np.array([1.0, 0.5, -1.0, 0.0] * 4, np.float32), (1, 2))
    small[0, 16] = 6.0
    packed, scales, gs = o.quantize(bits_of(small))
    assert o.unpack_codes(packed)[0, 0] == 7


def check_zero_cases(o):
    z = np.zeros((3, 32), dtype=np.uint16)
    packed, scales, gs = o.quantize(z)
    assert np.float32(gs).view(np.uint32) == np.float32(1e-12).view(np.uint32)
    assert not packed.any() and not scales.any()
    negz = np.full((2, 16), 0x8000, dtype=np.uint16)
    packed, scales, gs = o.quantize(negz)
    assert not packed.any() and not scales.any()
    w = wl.random_weight_bits(4, 64, seed=3)
    w[1, 16:32] = 0
    w[2, :16] = 0x8000
    packed, scales, gs = o.quantize(w)
    assert scales[1, 1] == 0 and not packed[1, 8:16].any()
    assert scales[2, 0] == 0 and not packed[2, :8].any()


def brute_quantize_scalar(w_f32_row, gs):
    """Element-by-element quantizer built from searches (tiny inputs only)."""
    inv = F32(1.0) / F32(gs)
    k = len(w_f32_row)
    scales, codes = [], []
    for j in range(k // 16):
        blk = [F32(v) for v in w_f32_row[16 * j:16 * j + 16]]
        b = max(abs(v) for v in blk)
        u = min(F32(F32(b) / F32(6.0)) * inv, F32(448.0))
        sb = int(brute_e4m3(np.array([u]))[0])
        s = F32(float(E4M3[sb]))
        r = F32(inv / s) if s > 0 else F32(0.0)
        scales.append(sb)
        for v in blk:
            q = F32(v * r)
            m = int(brute_e2m1(np.array([min(abs(float(q)), 6.0)]))[0])
            codes.append(m | (8 if (q < 0 and m != 0) else 0))
    return scales, codes


def check_tiny_bruteforce(o):
    rng = np.random.default_rng(9)
    for (n, k) in [(1, 16), (3, 32), (4, 64)]:
        w = wl.random_weight_bits(n, k, sigma=0.5, seed=n)
        # plant exact ties: values whose q lands on E2M1 midpoints in block 0 of row 0
        amax_row = wl.bf16_bits_to_f32(w)
        w[0, :8] = bits_of(np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32) * np.float32(0.25))
        w[0, 8:16] = bits_of(-np.abs(amax_row[0, 8:16]) * 0.01)
        packed, scales, gs = o.quantize(w)
        codes = o.unpack_codes(packed)
        wf = wl.bf16_bits_to_f32(w)
        for r in range(n):
            s_b, c_b = brute_quantize_scalar(wf[r], gs)
            assert scales[r].tolist() == s_b
            assert codes[r].tolist() == c_b
        assert rng is not None


def check_gemm_exact_rational(o):
    """fp64 GEMM reference against exact rational sums (within fp64 rounding)."""
    w = wl.random_weight_bits(3, 32, sigma=0.3, seed=1)
    x = wl.random_activation_bits(2, 32, seed=1)
    bias = wl.bias_bits(3, seed=2)
    packed, scales, gs = o.quantize(w)
    y = o.gemm_ref(x, packed, scales, gs, bias)
    codes = o.unpack_codes(packed)
    xf = wl.bf16_bits_to_f32(x)
    bf = wl.bf16_bits_to_f32(bias)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for kk in range(32):
                c = int(codes[n, kk])
                d = -grid[c & 7] if c & 8 else grid[c & 7]
                acc += Fraction(float(xf[m, kk])) * d * E4M3[int(scales[n, kk // 16])]
            acc = acc * Fraction(float(gs)) + Fraction(float(bf[n]))
            assert abs(Fraction(float(y[m, n])) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def check_gemm_onehot(o):
    w = wl.random_weight_bits(40, 64, sigma=0.05, seed=4)
    packed, scales, gs = o.quantize(w)
    codes = o.unpack_codes(packed)
    for kk in [0, 17, 63]:
        x = np.zeros((1, 64), dtype=np.uint16)
        x[0, kk] = 0x3F80   # 1.0
        y = o.gemm_ref(x, packed, scales, gs)[0]
        grid = np.array(E2M1_GRID)
        d = np.where(codes[:, kk] & 8, -1.0, 1.0) * grid[codes[:, kk] & 7]
        s = np.array([float(E4M3[int(b)]) for b in scales[:, kk // 16]])
        assert np.array_equal(y, d * s * float(gs))


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def facts(golden_dir):
    return load(golden_dir, "page_facts.json")


@pytest.fixture(scope="module")
def worked(golden_dir):
    return load(golden_dir, "worked_example.json")


def test_page_constants(facts):
    assert O.E4M3_MAX == facts["fp8_max"]["value"] == float(torch.finfo(torch.float8_e4m3fn).max)
    assert O.E2M1_MAX == facts["global_scale"]["e2m1_max"]
    assert O.GS_DIVISOR == facts["gs_divisor"]["value"] == O.E2M1_MAX * O.E4M3_MAX
    assert O.GROUP == facts["group_size"]["value"]


def test_code_table(facts):
    check_code_table(O, facts)


def test_decode_all_16_codes(facts):
    vals = O.e2m1_value(np.arange(16, dtype=np.uint8))
    dm = facts["e2m1_code_table"]["doubled_magnitudes"]
    assert vals[:8].tolist() == [d / 2 for d in dm]
    assert vals[8:].tolist() == [-d / 2 for d in dm]


def test_sign_and_zero(facts):
    check_sign_and_zero(O, facts)


def test_packing(facts):
    check_packing(O, facts)


def test_worked_example(worked):
    check_worked_example(O, worked)


def test_global_scale_exhaustive():
    check_gs_exhaustive(O)


def test_global_scale_closed_forms():
    check_gs_closed_forms(O)


def test_e4m3_decode_definition():
    check_e4m3_decode(O)


def test_e4m3_rne_bruteforce():
    check_e4m3_bruteforce(O)


def test_e4m3_rne_matches_torch_cast():
    """The library cast the quantizer on the page applies to its block scales."""
    u = e4m3_probe_inputs()
    ours = O.e4m3_encode_rne(u)
    theirs = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
    # the constructed tie: amax 2688 (gs = 1), block max 6.375 -> u = 1.0625 -> 1.0
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 2688.0
    w[0, 16] = 6.375
    _, scales, gs = O.quantize(bits_of(w))
    assert gs == F32(1.0) and scales[0, 1] == 0x38


def test_e4m3_full_sweep_of_sampled_exponents():
    """Every float32 of [2^-12, 448] in a 1/256 sample of mantissas, against torch."""
    mant = np.arange(0, 1 << 23, 256, dtype=np.uint32)
    exps = np.arange(127 - 12, 127 + 9, dtype=np.uint32)
    u = ((exps[:, None] << 23) | mant[None, :]).reshape(-1).view(np.float32)
    u = u[u <= 448]
    ours = O.e4m3_encode_rne(u)
    theirs = torch.from_numpy(u.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e2m1_rne_bruteforce():
    check_e2m1_bruteforce(O)


def test_block_max_invariant():
    for seed, sigma in [(0, 0.02), (1, 1.0), (2, 30.0)]:
        check_block_max_invariant(O, wl.random_weight_bits(64, 256, sigma=sigma, seed=seed))


def test_dequant_error_bound():
    check_dequant_error_bound(O, wl.random_weight_bits(64, 256, sigma=0.02, seed=6))


def test_grid_roundtrip():
    check_grid_roundtrip(O)


def test_heavy_grid_row_keeps_its_codes():
    """The heavy-tailed workload's grid row quantizes to exactly the generator's codes."""
    k = 7168
    w = wl.random_weight_bits(4, k, sigma=0.01, seed=8)
    w[0, 5] = bits_of([12.6875])[0]        # an amax like the heavy-tailed tensor's
    w[3] = wl.grid_row_bits(k)
    packed, scales, gs = O.quantize(w)
    g = wl.bf16_bits_to_f32(wl.grid_row_bits(k)).astype(np.float64)
    want = brute_e2m1(np.abs(g)) | np.where(g < 0, 8, 0).astype(np.uint8)
    want = np.where((want & 7) == 0, 0, want)
    assert np.array_equal(O.unpack_codes(packed)[3], want)
    assert np.all(O.e4m3_value(scales[3]) >= 2.0 ** -6)


def test_zero_cases():
    check_zero_cases(O)


def test_tiny_bruteforce():
    check_tiny_bruteforce(O)


def test_gemm_exact_rational():
    check_gemm_exact_rational(O)


def test_gemm_onehot():
    check_gemm_onehot(O)


def test_quantize_rows_is_row_local():
    w = wl.random_weight_bits(50, 128, sigma=0.1, seed=2)
    packed, scales, gs = O.quantize(w)
    p, s = O.quantize_rows(w[17:23], gs)
    assert np.array_equal(p, packed[17:23]) and np.array_equal(s, scales[17:23])


def test_contract_errors():
    with pytest.raises(O.OracleContractError):
        O.quantize(np.zeros((2, 24), np.uint16))
    with pytest.raises(O.OracleContractError):
        O.quantize(np.zeros((0, 16), np.uint16))
    w = np.zeros((1, 16), np.uint16)
    w[0, 3] = 0x7F80   # +inf
    with pytest.raises(O.OracleContractError):
        O.quantize(w)


def test_argmax_agreement_tie_rule():
    y64 = np.array([[1.0, 1.0000001, 0.5], [3.0, 2.0, 1.0]])
    ybf = np.array([[1.0, 1.0, 0.5], [3.0, 2.0, 1.0]])   # row 0: tie in bf16
    tie, strict = O.argmax_agreement(ybf, y64)
    assert tie == 1.0 and strict == 0.5


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

def mutant(**overrides):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in vars(O).items() if not k.startswith("__")})
    for name, fn in overrides.items():
        m.__dict__[name] = fn
    # functions look up globals in their own module: rebind them to the mutant
    for name, obj in list(m.__dict__.items()):
        if isinstance(obj, types.FunctionType) and name not in overrides:
            m.__dict__[name] = types.FunctionType(obj.__code__, m.__dict__, name, obj.__defaults__, obj.__closure__)
    return m


def _pins_fail(o, facts, worked):
    checks = [
        lambda: check_code_table(o, facts),
        lambda: check_packing(o, facts),
        lambda: check_worked_example(o, worked),
        lambda: check_gs_closed_forms(o),
        lambda: check_e4m3_bruteforce(o),
        lambda: check_e2m1_bruteforce(o),
        lambda: check_zero_cases(o),
        lambda: check_tiny_bruteforce(o),
        lambda: check_gemm_exact_rational(o),
        lambda: check_gemm_onehot(o),
        lambda: check_grid_roundtrip(o),
        lambda: check_dequant_error_bound(o, wl.random_weight_bits(16, 64, sigma=0.02, seed=6)),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, Exception):
            failed += 1
    return failed


def _pack_high_first(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 1::2] | (codes[:, 0::2] << 4)).astype(np.uint8)


def _e4m3_truncate(u):
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    out = np.zeros(u.shape, dtype=np.int64)
    sub = u < 2.0 ** -6
    out[sub] = np.floor(u[sub] * 512).astype(np.int64)
    mant, exp = np.frexp(u[~sub])
    out[~sub] = ((exp - 1 + 7) << 3) + np.floor((2 * mant - 1) * 8).astype(np.int64)
    return out.astype(np.uint8)


def _e2m1_ties_away(a):
    a = np.asarray(a, dtype=np.float32)
    code = np.zeros(a.shape, dtype=np.uint8)
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        code += (a >= np.float32(t))
    return code


def _gs_wrong_divisor(amax):
    return max(np.float32(np.float32(amax) / np.float32(6.0)), np.float32(1e-12))


def _element_codes_sign_on_zero(w_rows_f32, s_vals, inv_gs):
    n, k = w_rows_f32.shape
    safe = np.where(s_vals > 0, s_vals, np.float32(1.0)).astype(np.float32)
    r = np.where(s_vals > 0, np.float32(inv_gs) / safe, np.float32(0.0)).astype(np.float32)
    q = (w_rows_f32.reshape(n, k // 16, 16) * r[:, :, None]).astype(np.float32).reshape(n, k)
    mag = e2m1_code_ref(np.minimum(np.abs(q), np.float32(6.0)))
    return (mag | ((np.signbit(q)).astype(np.uint8) << 3)).astype(np.uint8)


def e2m1_code_ref(a):
    return brute_e2m1(np.asarray(a).reshape(-1)).reshape(np.shape(a))


def _dequant_no_gs(packed, scales, gs):
    codes = O.unpack_codes(packed)
    n, k = codes.shape
    d = O.e2m1_value(codes).reshape(n, k // 16, 16)
    return (d * O.e4m3_value(scales)[:, :, None]).reshape(n, k)


def _block_scales_no_inv(w_rows_f32, inv_gs):
    n, k = w_rows_f32.shape
    b = np.abs(w_rows_f32.reshape(n, k // 16, 16)).max(axis=2).astype(np.float32)
    u = np.minimum(b / np.float32(6.0), np.float32(448.0))
    s_bytes = _e4m3_ref(u)
    return s_bytes, O.e4m3_value(s_bytes).astype(np.float32)


def _e4m3_ref(u):
    return brute_e4m3(np.asarray(u, dtype=np.float32).reshape(-1)).reshape(np.shape(u))


@pytest.mark.parametrize("name,overrides", [
    ("pack high nibble first", {"pack_codes": _pack_high_first}),
    ("e4m3 truncation", {"e4m3_encode_rne": _e4m3_truncate}),
    ("e2m1 ties away from zero", {"e2m1_magnitude_code": _e2m1_ties_away}),
    ("global scale divides by 6 only", {"global_scale": _gs_wrong_divisor}),
    ("sign bit on -0 / rounded zero", {"element_codes": _element_codes_sign_on_zero}),
    ("dequant drops gs", {"dequantize": _dequant_no_gs}),
    ("block scale ignores inv_gs", {"block_scales": _block_scales_no_inv}),
])
def test_planted_mistakes_are_caught(name, overrides, facts, worked):
    assert _pins_fail(O, facts, worked) == 0
    assert _pins_fail(mutant(**overrides), facts, worked) >= 1, name


def _sweep_float32(top_value, chunk, fn):
    """Run ``fn`` over every non-negative float32 up to ``top_value`` (bit
    patterns 0 .. bits(top_value)) in chunks on a thread pool; returns the
    summed counts ``fn`` reports."""
    import concurrent.futures

    top = int(np.float32(top_value).view(np.uint32))

    def work(c0):
        u = np.arange(c0, min(top + 1, c0 + chunk), dtype=np.uint32).view(np.float32)
        return fn(u)

    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        return sum(ex.map(work, range(0, top + 1, chunk)))


@pytest.mark.slow
def test_e4m3_rne_exhaustive_against_torch_cast():
    """Every float32 of [0, 448] (1.14e9 values): the oracle's E4M3 rounding
    equals torch's float8_e4m3fn cast, the cast the page applies."""
    def bad(u):
        theirs = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return int(np.count_nonzero(O.e4m3_encode_rne(u) != theirs))

    threads = torch.get_num_threads()
    torch.set_num_threads(1)                         # the sweep's own threads split the work
    try:
        assert _sweep_float32(448.0, 1 << 22, bad) == 0
    finally:
        torch.set_num_threads(threads)


@pytest.mark.slow
def test_e2m1_rne_exhaustive_against_search():
    """Every float32 of [0, 6] (1.09e9 values): the oracle's interval form of
    E2M1 rounding equals the nearest-grid-value search with ties to even."""
    def bad(u):
        return int(np.count_nonzero(O.e2m1_magnitude_code(u) != brute_e2m1(u)))

    assert _sweep_float32(6.0, 1 << 20, bad) == 0
