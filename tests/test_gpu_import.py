"""GPU parity of the checkpoint-import calls against the import oracle.

nvfp4_fill_scale_sentinel must leave every block-scale byte at 0x7F;
nvfp4_import_checkpoint must give the oracle's global scale bit for bit and
the oracle's flags for every case; and a checkpoint made of several
partitions, quantized by the oracle with their own global scales and stored
in either convention, must give through nvfp4_w4a16_gemm the oracle's logits
for the collapsed global scale (decode and prefill kernels).
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_import_oracle as I
import oracle.nvfp4_oracle as O
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, check_gemm, dev_u8, f32_bits, gemm_gpu

pytestmark = pytest.mark.gpu

CONVS = (I.MODELOPT, I.COMPRESSED_TENSORS)


def run_import(part, scale_bytes, k, conv):
    ps = torch.from_numpy(np.asarray(part, np.float32).copy()).to(DEV)
    gs, flags = B.nvfp4_import_checkpoint(ps, dev_u8(scale_bytes), k, conv)
    torch.cuda.synchronize()
    return np.float32(gs.item()), int(flags.item())


def assert_report(part, scale_bytes, k, conv, label=""):
    gs, flags = run_import(part, scale_bytes, k, conv)
    want_gs, want_flags = I.import_report(np.asarray(part, np.float32), scale_bytes, conv)
    assert f32_bits(gs) == f32_bits(want_gs), f"{label}: gs {gs!r} != {want_gs!r}"
    assert flags == want_flags, f"{label}: flags {flags} != {want_flags}"
    return gs, flags


def finite_scale_bytes(rng, n, k):
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    return rng.choice(finite, size=(n, k // 16))


@pytest.mark.parametrize("n,k", [(3, 16), (1027, 48), (4096, 512), (129, 7168)])
def test_fill_sentinel_marks_every_byte(n, k):
    s = torch.zeros((n, k // 16), dtype=torch.uint8, device=DEV)
    B.nvfp4_fill_scale_sentinel(s, k)
    torch.cuda.synchronize()
    assert bool((s == 0x7F).all())
    for conv in CONVS:
        _, flags = assert_report([2e-4], s.cpu().numpy(), k, conv, "sentinel")
        assert flags & I.FLAG_SCALES_NOT_LOADED


@pytest.mark.parametrize("n,k", [(3, 16), (1027, 48), (4096, 512), (129, 7168)])
@pytest.mark.parametrize("where", ["none", "first", "middle", "last", "last16"])
@pytest.mark.parametrize("nan_byte", [0x7F, 0xFF])
def test_nan_scan_finds_a_single_unloaded_scale(n, k, where, nan_byte):
    rng = np.random.default_rng(n + k)
    s = finite_scale_bytes(rng, n, k)
    flat = s.reshape(-1)
    pos = {"none": None, "first": 0, "middle": flat.size // 2, "last": flat.size - 1,
           "last16": max(0, (flat.size // 16) * 16 - 1)}[where]
    if pos is not None:
        flat[pos] = nan_byte
    assert_report([1e-3], s, k, I.MODELOPT, f"{n}x{k} {where}")


@pytest.mark.parametrize("conv", CONVS)
@pytest.mark.parametrize("p", [1, 3, 64, 65, 200])
def test_global_scale_of_random_partitions(conv, p):
    rng = np.random.default_rng(7 * p)
    gs_i = np.float32(rng.uniform(1e-5, 1e-2, size=p)).astype(np.float32)
    part = I.checkpoint_partition_scales(gs_i, conv)
    s = finite_scale_bytes(rng, 64, 256)
    gs, flags = assert_report(part, s, 256, conv, f"{conv} P={p}")
    assert (flags & I.FLAG_PARTITIONS_DIFFER) == (I.FLAG_PARTITIONS_DIFFER if p > 1 else 0)


@pytest.mark.parametrize("conv", CONVS)
@pytest.mark.parametrize("part", [[0.0], [-1e-3], [float("inf")], [float("nan")], [1e-3, float("nan"), 2e-3],
                                  [0.0, -0.0], [-0.0, 0.0], [3e-3, 3e-3, 3e-3], [1e-40], [3.0e38, 1.0]])
def test_special_partition_scales(conv, part):
    s = np.zeros((16, 1), np.uint8)
    assert_report(part, s, 16, conv, f"{conv} {part}")


@pytest.mark.parametrize("conv", CONVS)
@pytest.mark.parametrize("m", [4, 40, 130])
def test_gemm_on_an_imported_three_partition_checkpoint(conv, m):
    """Partitions of rows with their own amax (as a fused q/k/v would have),
    quantized by the oracle each with its own global scale, stored in the
    convention, imported on the GPU; the GEMM then uses the collapsed scale."""
    k = 512
    parts = [wl.random_weight_bits(rows, k, sigma=sig, seed=40 + i)
             for i, (rows, sig) in enumerate([(300, 0.02), (129, 0.05), (211, 0.01)])]
    quant = [O.quantize(wb) for wb in parts]
    packed = np.concatenate([q[0] for q in quant])
    scales = np.concatenate([q[1] for q in quant])
    gs_i = np.array([q[2] for q in quant], np.float32)
    stored = I.checkpoint_partition_scales(gs_i, conv)
    # the loader writes the block scales into a sentinel-filled buffer
    sd = torch.empty(scales.shape, dtype=torch.uint8, device=DEV)
    B.nvfp4_fill_scale_sentinel(sd, k)
    sd.copy_(dev_u8(scales))
    gs_dev, flags = B.nvfp4_import_checkpoint(torch.from_numpy(stored).to(DEV), sd, k, conv)
    torch.cuda.synchronize()
    want_gs, want_flags = I.import_report(stored, scales, conv)
    assert f32_bits(gs_dev.item()) == f32_bits(want_gs)
    assert int(flags.item()) == want_flags == I.FLAG_PARTITIONS_DIFFER
    with pytest.warns(UserWarning):
        B.check_import_flags(flags)
    x = wl.random_activation_bits(m, k, seed=50 + m)
    y = gemm_gpu(x, (dev_u8(packed), sd, gs_dev))
    check_gemm(y, x, packed, scales, want_gs, label=f"{conv} M={m}")


def test_check_import_flags_rejects_unloaded_scales():
    s = torch.empty((8, 2), dtype=torch.uint8, device=DEV)
    B.nvfp4_fill_scale_sentinel(s, 32)
    _, flags = B.nvfp4_import_checkpoint(torch.ones(1, device=DEV) * 1e-3, s, 32, "modelopt")
    with pytest.raises(B.NVFP4NotLoadedError):
        B.check_import_flags(flags)


def test_full_size_scan_of_the_8b_shape_scales():
    """128256 x 4096 weight: 32.8 MB of block scales, one NaN in the last byte."""
    n, k = 128256, 4096
    rng = np.random.default_rng(5)
    s = finite_scale_bytes(rng, n, k)
    assert_report([1e-3], s, k, I.MODELOPT, "8B clean")
    s[-1, -1] = 0xFF
    assert_report([1e-3], s, k, I.MODELOPT, "8B last byte")
