"""C-ABI boundary checks that need no GPU.

The library must load, export every entry point the header declares, and
reject bad arguments with the documented status before it makes any HIP call
(so these calls are safe without a device; the pointers below are never
dereferenced).
"""

import ctypes
import os
import re
import subprocess

import pytest

from nvfp4_w4a16_lm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_w4a16.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ALIAS, ERR_ARG, ERR_SCRATCH = 0, 1, 2, 3, 4, 6, 7

# Fake, well-separated, 256-byte aligned addresses: only compared, never touched.
W, P, S, G, X, Y, B = (0x10000000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status|const char\*|int|int64_t)\s+(nvfp4_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    path = binding.library_path()
    if not os.path.exists(path):
        pytest.fail(f"library not built: {path} (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_the_three_calls_and_the_checkpoint_calls():
    fns = declared_functions()
    for name in ("nvfp4_quantize", "nvfp4_refresh_inplace", "nvfp4_w4a16_gemm",
                 "nvfp4_fill_scale_sentinel", "nvfp4_import_checkpoint"):
        assert name in fns
    assert set(fns) == set(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == binding.ABI_VERSION
    for st in range(8):
        assert lib.nvfp4_status_string(st).decode()
    assert lib.nvfp4_status_string(99).decode() == "unknown status"
    assert lib.nvfp4_last_hip_error().decode() == ""


def q(lib, w=W, n=1024, k=512, p=P, s=S, g=G, fn="nvfp4_quantize"):
    return getattr(lib, fn)(w, n, k, p, s, g, None)


@pytest.mark.parametrize("fn", ["nvfp4_quantize", "nvfp4_refresh_inplace"])
def test_quantize_validation(lib, fn):
    assert q(lib, w=0, fn=fn) == ERR_NULL
    assert q(lib, p=0, fn=fn) == ERR_NULL
    assert q(lib, s=0, fn=fn) == ERR_NULL
    assert q(lib, g=0, fn=fn) == ERR_NULL
    # K must be a positive multiple of 16 (KNvfp4Static in vLLM modelopt.py rejects others)
    for n, k in [(0, 512), (-1, 512), (4, 0), (4, 8), (4, 24), (4, 520), (4, -16), (1 << 31, 16)]:
        assert q(lib, n=n, k=k, fn=fn) == ERR_SHAPE, (n, k)
    assert q(lib, w=W + 8, fn=fn) == ERR_ALIGN
    assert q(lib, p=P + 4, fn=fn) == ERR_ALIGN
    assert q(lib, s=S + 2, fn=fn) == ERR_ALIGN
    assert q(lib, g=G + 2, fn=fn) == ERR_ALIGN
    # outputs overlapping the weight or each other
    assert q(lib, p=W + 1024, fn=fn) == ERR_ALIAS
    assert q(lib, s=P + 16, fn=fn) == ERR_ALIAS
    assert q(lib, g=S + 64, fn=fn) == ERR_ALIAS
    assert q(lib, g=P, fn=fn) == ERR_ALIAS
    # the weight ends exactly where packed starts: no overlap, but we stop before HIP by
    # making another argument invalid
    assert q(lib, p=W + 1024 * 512 * 2, g=0, fn=fn) == ERR_NULL


def gm(lib, x=X, m=4, k=512, p=P, s=S, g=G, n=1024, b=0, y=Y):
    return lib.nvfp4_w4a16_gemm(x, m, k, p, s, g, n, b, y, None)


def test_gemm_validation(lib):
    assert gm(lib, x=0) == ERR_NULL
    assert gm(lib, p=0) == ERR_NULL
    assert gm(lib, s=0) == ERR_NULL
    assert gm(lib, g=0) == ERR_NULL
    assert gm(lib, y=0) == ERR_NULL
    for m, k, n in [(-1, 512, 1024), (4, 8, 1024), (4, 40, 1024), (4, 512, 0), (4, 512, -3)]:
        assert gm(lib, m=m, k=k, n=n) == ERR_SHAPE, (m, k, n)
    assert gm(lib, x=X + 2) == ERR_ALIGN
    assert gm(lib, y=Y + 8) == ERR_ALIGN
    assert gm(lib, p=P + 8) == ERR_ALIGN
    assert gm(lib, s=S + 1) == ERR_ALIGN
    assert gm(lib, g=G + 1) == ERR_ALIGN
    assert gm(lib, b=B + 1) == ERR_ALIGN
    assert gm(lib, y=X) == ERR_ALIAS
    assert gm(lib, y=P + 256) == ERR_ALIAS
    assert gm(lib, y=S - 16) == ERR_ALIAS
    assert gm(lib, y=G - 64) == ERR_ALIAS
    assert gm(lib, b=B, y=B - 32) == ERR_ALIAS
    # M == 0 is an empty GEMM: validated, nothing enqueued, no HIP call; x and y
    # may be NULL then (empty tensors have no storage)
    assert gm(lib, m=0) == OK
    assert gm(lib, m=0, x=0, y=0) == OK
    assert gm(lib, m=1, x=0) == ERR_NULL


def imp(lib, ps=P, np_=3, conv=0, s=S, n=1024, k=512, g=G, f=B):
    return lib.nvfp4_import_checkpoint(ps, np_, conv, s, n, k, g, f, None)


def test_import_checkpoint_validation(lib):
    assert imp(lib, ps=0) == ERR_NULL
    assert imp(lib, s=0) == ERR_NULL
    assert imp(lib, g=0) == ERR_NULL
    assert imp(lib, f=0) == ERR_NULL
    assert imp(lib, conv=2) == ERR_ARG
    assert imp(lib, conv=-1) == ERR_ARG
    for np_, n, k in [(0, 1024, 512), (-1, 1024, 512), ((1 << 20) + 1, 1024, 512), (3, 0, 512), (3, 1024, 40)]:
        assert imp(lib, np_=np_, n=n, k=k) == ERR_SHAPE, (np_, n, k)
    assert imp(lib, ps=P + 2) == ERR_ALIGN
    assert imp(lib, s=S + 4) == ERR_ALIGN       # the scan reads 16-byte vectors
    assert imp(lib, g=G + 1) == ERR_ALIGN
    assert imp(lib, f=B + 2) == ERR_ALIGN
    assert imp(lib, g=S + 1024) == ERR_ALIAS
    assert imp(lib, f=P + 8) == ERR_ALIAS
    assert imp(lib, g=G, f=G) == ERR_ALIAS
    assert lib.nvfp4_fill_scale_sentinel(0, 1024, 512, None) == ERR_NULL
    assert lib.nvfp4_fill_scale_sentinel(S, 1024, 40, None) == ERR_SHAPE
    assert lib.nvfp4_fill_scale_sentinel(S + 4, 1024, 512, None) == ERR_ALIGN


def test_fp8_validation(lib):
    q8 = lib.nvfp4_fp8_quantize_rows
    assert q8(0, 1024, 512, P, S, None) == ERR_NULL
    assert q8(W, 1024, 40, P, S, None) == ERR_SHAPE
    assert q8(W + 8, 1024, 512, P, S, None) == ERR_ALIGN
    assert q8(W, 1024, 512, P + 8, S, None) == ERR_ALIGN
    assert q8(W, 1024, 512, W + 4096, S, None) == ERR_ALIAS
    g8 = lib.nvfp4_fp8_gemm
    assert g8(0, G, 4, 512, P, S, 1024, None, Y, None) == ERR_NULL
    assert g8(0, 0, 0, 512, P, S, 1024, None, 0, None) == OK
    assert g8(X, G, 4, 40, P, S, 1024, None, Y, None) == ERR_SHAPE
    assert g8(X, G, -1, 512, P, S, 1024, None, Y, None) == ERR_SHAPE
    assert g8(X + 8, G, 4, 512, P, S, 1024, None, Y, None) == ERR_ALIGN
    assert g8(X, G, 4, 512, P, S, 1024, B + 1, Y, None) == ERR_ALIGN
    assert g8(X, G, 4, 512, P, S, 1024, None, P + 256, None) == ERR_ALIAS


def test_w4a4_validation(lib):
    qa = lib.nvfp4_quantize_activations
    assert qa(0, 4, 512, G, P, S, None) == ERR_NULL
    assert qa(X, 4, 40, G, P, S, None) == ERR_SHAPE
    assert qa(X, 0, 512, G, P, S, None) == ERR_SHAPE
    assert qa(X + 8, 4, 512, G, P, S, None) == ERR_ALIGN
    assert qa(X, 4, 512, G, P, X + 64, None) == ERR_ALIAS
    assert lib.nvfp4_w4a4_workspace_bytes(4, 512) == 2 * 4 * 512 + 16
    g4 = lib.nvfp4_w4a4_gemm
    args = dict(xp=X, xs=B, gi=G + 64, m=4, k=512, p=P, s=S, g=G, n=1024, b=None, ws=W, y=Y)

    def call(**kw):
        a = {**args, **kw}
        return g4(a["xp"], a["xs"], a["gi"], a["m"], a["k"], a["p"], a["s"], a["g"], a["n"], a["b"], a["ws"],
                  a["y"], None)
    assert call(ws=0) == ERR_NULL
    assert call(m=0, xp=0, xs=0, gi=0, ws=0, y=0) == OK
    assert call(k=40) == ERR_SHAPE
    assert call(ws=W + 8) == ERR_ALIGN
    assert call(ws=Y + 64) == ERR_ALIAS
    assert call(ws=P - 1024) == ERR_ALIAS
    assert call(y=X + 256) == ERR_ALIAS
    # the no-allocation variant: same checks without a workspace, plus the size of its static scratch
    gn = lib.nvfp4_w4a4_gemm_noalloc

    def call_n(**kw):
        a = {**args, **kw}
        return gn(a["xp"], a["xs"], a["gi"], a["m"], a["k"], a["p"], a["s"], a["g"], a["n"], a["b"], a["y"], None)
    assert call_n(y=0) == ERR_NULL
    assert call_n(m=0, xp=0, xs=0, gi=0, y=0) == OK
    assert call_n(k=40) == ERR_SHAPE
    assert call_n(y=Y + 8) == ERR_ALIGN
    assert call_n(y=X + 256) == ERR_ALIAS
    # 2 M K + 16 bytes must fit the 4 MiB array: M K <= 2097144
    assert lib.nvfp4_w4a4_workspace_bytes(2048, 1024) > binding.W4A4_SCRATCH_BYTES
    assert call_n(m=2048, k=1024) == ERR_SCRATCH
    assert call_n(m=2048, k=1024, y=X + 256) == ERR_SCRATCH      # size is checked before aliasing


def test_binding_import_rejects_unknown_convention():
    import torch
    with pytest.raises(ValueError):
        binding.nvfp4_import_checkpoint(torch.ones(1), torch.zeros(4, 2, dtype=torch.uint8), 32, "gguf")


def test_binding_maps_shape_errors_to_valueerror(lib):
    with pytest.raises(ValueError):
        binding._check("nvfp4_quantize", ERR_SHAPE)
    with pytest.raises(binding.NVFP4Error):
        binding._check("nvfp4_quantize", ERR_ALIAS)


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no CPU path."""
    pkg = os.path.join(ROOT, "nvfp4_w4a16_lm_amd")
    for fname in os.listdir(pkg):
        if fname.endswith(".py"):
            text = open(os.path.join(pkg, fname)).read()
            assert "oracle" not in text.replace("the oracle", ""), fname


def test_moe_validation(lib):
    """Mixture-of-experts calls reject bad arguments before any HIP call."""
    assert lib.nvfp4_moe_gemm_workspace_bytes(10, 8) == 4 * (12 + 12)
    assert lib.nvfp4_moe_gemm_workspace_bytes(-1, 8) == 0
    T, k, E, H, I = 5, 2, 8, 512, 256
    npairs = T * k
    assert lib.nvfp4_moe_workspace_bytes(T, k, E, H, I) == 256 + 256 * ((npairs * 4 * I + 255) // 256) + \
        256 * ((npairs * 2 * I + 255) // 256) + 256 * ((npairs * 2 * H + 255) // 256)
    g = lib.nvfp4_moe_w4a16_gemm
    base = dict(x=X, rows=T, K=H, ids=B, P=npairs, div=k, p=P, s=S, g=G, E=E, N=2 * I, ws=W, y=Y, inv=None)

    def call(**kw):
        a = {**base, **kw}
        return g(a["x"], a["rows"], a["K"], a["ids"], a["P"], a["div"], a["p"], a["s"], a["g"], a["E"], a["N"],
                 a["ws"], a["y"], a["inv"], None)
    assert call(ids=0) == ERR_NULL
    assert call(ws=0) == ERR_NULL
    assert call(P=0, x=0, ids=0, ws=0, y=0) == OK
    assert call(K=40) == ERR_SHAPE
    assert call(E=0) == ERR_SHAPE
    assert call(E=65535) == ERR_SHAPE                       # the grid holds E + 1 expert rows
    assert call(div=0) == ERR_SHAPE
    assert call(rows=T - 1) == ERR_SHAPE                     # x_rows < ceil(P / row_div)
    assert call(x=X + 8) == ERR_ALIGN
    assert call(ids=B + 2) == ERR_ALIGN
    assert call(y=X + 256) == ERR_ALIAS
    assert call(ws=Y + 64) == ERR_ALIAS
    assert lib.nvfp4_moe_silu_and_mul(X, 4, 12, Y, None) == ERR_SHAPE
    assert lib.nvfp4_moe_silu_and_mul(X, 4, 16, X + 64, None) == ERR_ALIAS
    assert lib.nvfp4_moe_silu_and_mul(X + 2, 4, 16, Y, None) == ERR_ALIGN
    assert lib.nvfp4_moe_combine(X, G, 3, 0, 64, Y, None) == ERR_SHAPE
    assert lib.nvfp4_moe_combine(X, G, 3, 2, 64, X + 128, None) == ERR_ALIAS
    f = lib.nvfp4_moe_w4a16_forward
    assert f(X, T, H, B, G + 4096, k, P, S, G, W + 4096, S + 4096, G + 8192, E, 40, W, Y, None, None) == ERR_SHAPE
    assert f(X, T, H, B, G + 4096, k, P, S, G, W + 4096, S + 4096, G + 8192, E, I, 0, Y, None, None) == ERR_NULL


def test_binding_collapses_w13_scale2_to_the_w1_column():
    """ModelOpt's fused w13 keeps one global scale per expert, the w1 column,
    with a warning when the w3 column differs (host logic, CPU tensors)."""
    import warnings

    import torch
    same = torch.tensor([[0.5, 0.5], [0.25, 0.25]], dtype=torch.float32)
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        assert torch.equal(binding.moe_collapse_w13_scale2(same), torch.tensor([0.5, 0.25]))
    differ = torch.tensor([[0.5, 0.5], [0.25, 0.375]], dtype=torch.float32)
    with pytest.warns(UserWarning):
        got = binding.moe_collapse_w13_scale2(differ)
    assert torch.equal(got, torch.tensor([0.5, 0.25]))
