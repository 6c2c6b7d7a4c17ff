"""GPU proof that the hardware converters the kernels use follow the oracle's rules.

Encode (vLLM API docs, quantization.online.lm_head, _quantize_nvfp4: the E2M1
code table and the sign rule ``values < 0``): the quantizer rounds every
q = w * r with gfx950's fp32 -> fp4 converter and clears the sign of zero
codes (``fix_zero_signs``).  The sweep below runs that exact device code on
every float32 bit pattern with |q| <= 16 -- both signs, -0, subnormals, every
rounding threshold, the saturation above 6 and the largest q the quantizer can
produce (about 9, from a subnormal block scale) -- and compares each code with
the oracle's element step (``element_codes`` with scale 1, so q passes
through unchanged).

Dequantize: the fp32, f16 (both forms) and power-of-two bf16 routes the GEMM kernels use,
for all 256 code bytes under all 127 finite E4M3 scale bytes, against the
oracle's exact values of code * scale.
"""

import concurrent.futures
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libnvfp4_test_support.so")
TOP = int(np.float32(16.0).view(np.uint32))        # sweep bit patterns 0 .. TOP
CHUNK = 1 << 26                                     # values per GPU call
SUB = 1 << 22                                       # values per oracle call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.nvfp4_test_e2m1_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.nvfp4_test_dequant_table.argtypes = [ctypes.c_void_p] * 7
    lib.nvfp4_test_e4m3_bf16_table.argtypes = [ctypes.c_void_p] * 3
    return lib


def oracle_codes(first: int, count: int, sign: int) -> np.ndarray:
    q = (np.arange(first, first + count, dtype=np.uint32) | np.uint32(sign)).view(np.float32)
    rows = q.reshape(-1, 16)
    return O.element_codes(rows, np.ones((rows.shape[0], 1), np.float32), np.float32(1.0)).reshape(-1)


def gpu_codes(words: np.ndarray) -> np.ndarray:
    return np.stack([(words >> np.uint32(4 * j)) & np.uint32(0xF) for j in range(8)], axis=1).reshape(-1).astype(
        np.uint8)


def test_e2m1_encode_matches_oracle_on_every_float32_up_to_16(lib):
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty(CHUNK // 8, dtype=torch.int32, device="cuda")
    checked = 0
    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        for sign in (0, 0x80000000):
            for first in range(0, TOP + 1, CHUNK):
                count = min(CHUNK, (TOP + 1 - first + 15) // 16 * 16)
                rc = lib.nvfp4_test_e2m1_sweep(first, sign, count, out.data_ptr(), stream)
                assert rc == 0, f"sweep launch failed: {rc}"
                words = out[:count // 8].cpu().numpy().view(np.uint32)

                def cmp(off, first=first, sign=sign, words=words, count=count):
                    n = min(SUB, count - off)
                    got = gpu_codes(words[off // 8:(off + n) // 8])
                    want = oracle_codes(first + off, n, sign)
                    bad = np.flatnonzero(got != want)
                    if bad.size:
                        i = int(bad[0])
                        b = (first + off + i) | sign
                        return (f"{bad.size} mismatches from bits {first + off:#010x} (sign {sign:#x}); first: "
                                f"q = {np.uint32(b).view(np.float32)!r} ({b:#010x}) gpu code {got[i]:#x}, "
                                f"oracle {want[i]:#x}")
                    return None

                errs = [e for e in ex.map(cmp, range(0, count, SUB)) if e]
                assert not errs, errs[0]
                checked += count
    print(f"e2m1 encode: {checked} float32 values, 0 mismatches", flush=True)
    assert checked >= 2 * (TOP + 1)


def test_dequant_routes_exact_for_all_codes_and_scales(lib):
    stream = torch.cuda.current_stream().cuda_stream
    f32r = torch.empty(127 * 256, dtype=torch.int32, device="cuda")
    f16r = torch.empty_like(f32r)
    f16s = torch.empty_like(f32r)
    p2r = torch.empty_like(f32r)
    e2 = torch.empty(127, dtype=torch.float32, device="cuda")
    mu = torch.empty(127, dtype=torch.int16, device="cuda")
    rc = lib.nvfp4_test_dequant_table(f32r.data_ptr(), f16r.data_ptr(), f16s.data_ptr(), p2r.data_ptr(),
                                      e2.data_ptr(), mu.data_ptr(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    sbytes = np.arange(127, dtype=np.uint8)
    s = O.e4m3_value(sbytes)                                          # float64, exact
    cbytes = np.arange(256, dtype=np.uint8)
    codes = np.stack([cbytes & 0xF, cbytes >> 4], axis=1)             # low nibble first
    want = O.e2m1_value(codes)[None, :, :] * s[:, None, None]        # [scale, byte, pair]

    def halves(t, as_dtype):
        u = t.cpu().numpy().view(np.uint32).reshape(127, 256)
        pair = np.stack([u & 0xFFFF, u >> 16], axis=2).astype(np.uint16)
        if as_dtype == "bf16":
            return (pair.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return pair.view(np.float16).astype(np.float64)

    got32 = halves(f32r, "bf16")
    got16 = halves(f16r, "f16")
    assert np.array_equal(got32, want), "fp32-route (bf16) dequantization differs from code * scale"
    assert np.array_equal(got16, want), "f16-route dequantization differs from code * scale"
    assert np.array_equal(halves(f16s, "f16"), want), "f16 route with the scale as the converter's scale differs"
    # the power-of-two converter: code * e2 exactly, and e2 * mu == s
    e2h = e2.cpu().numpy().astype(np.float64)
    muh = mu.cpu().numpy().view(np.float16).astype(np.float64)
    assert np.array_equal(e2h * muh, s), "split_scale: e2 * mu != scale"
    nz = s > 0
    assert np.all((e2h[nz] == 2.0 ** np.floor(np.log2(s[nz]))) & (muh[nz] >= 1) & (muh[nz] < 2))
    got_p2 = halves(p2r, "bf16")
    want_p2 = O.e2m1_value(codes)[None, :, :] * e2h[:, None, None]
    assert np.array_equal(got_p2[nz], want_p2[nz]), "power-of-two bf16 converter differs from code * 2^e"
    assert np.all(np.isfinite(got_p2)), "a zero scale (e2 = 0) must still give finite values (they are times mu = 0)"
    # signs: negative codes give negative values, and code 8 (-0) gives a zero
    assert np.all(np.signbit(got32[:, 0x08, 0]) | (got32[:, 0x08, 0] == 0))


def test_e4m3_pair_to_bf16_exact_for_every_byte_pair(lib):
    """The FP8 dot kernel's converter (bytes 2 SEL, 2 SEL + 1 of a word -> two
    bf16): every pair of e4m3fn bytes, in both halves of a word, against the
    oracle's e4m3 decoding (vLLM modelopt.py, KFp8StaticChannel: the
    float8_e4m3fn format), rounded to bf16 (exact for every finite value);
    the NaN bytes 0x7F and 0xFF give NaN."""
    import oracle.fp8_oracle as F

    stream = torch.cuda.current_stream().cuda_stream
    lo = torch.empty(65536, dtype=torch.int32, device="cuda")
    hi = torch.empty_like(lo)
    assert lib.nvfp4_test_e4m3_bf16_table(lo.data_ptr(), hi.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    t = np.arange(65536, dtype=np.uint32)
    b = np.stack([t & 0xFF, t >> 8], axis=1).astype(np.uint8)          # [pair, element]
    nan = (b & 0x7F) == 0x7F
    want = np.where(nan, 0.0, F.e4m3_decode_signed(np.where(nan, 0, b)))
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want)   # exact in float32
    for name, got_t in (("low half", lo), ("high half", hi)):
        u = got_t.cpu().numpy().view(np.uint32)
        got = np.stack([(u & 0xFFFF) << 16, u & 0xFFFF0000], axis=1).astype(np.uint32).view(np.float32)
        assert np.all(np.isnan(got[nan])), f"{name}: NaN bytes"
        g, w = got[~nan].astype(np.float64), want[~nan]
        assert np.array_equal(g, w), f"{name}: {int(np.sum(g != w))} byte values differ"
