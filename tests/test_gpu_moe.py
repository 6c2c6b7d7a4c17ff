"""GPU parity of the W4A16 mixture-of-experts calls against
oracle/nvfp4_moe_oracle.py.

Grouped GEMM: every output of every pair against the fp64 reference on the
oracle's quantized experts, within the float32-accumulation bound plus one
bf16 rounding, and the norm bound; routing edge cases (experts with no
pair, more than one 64-pair block, ids outside [0, E), ragged K and N).
SiLU-and-mul and combine: every element on seeded inputs.  The whole layer:
every output within the oracle's propagated bound.
"""

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
import oracle.nvfp4_moe_oracle as MO
from nvfp4_w4a16_lm_amd import binding as B
from nvfp4_w4a16_lm_amd import workloads as wl

from gpu_util import DEV, dev_bf16, dev_u8, host_bits

pytestmark = pytest.mark.gpu


def experts(E, N, K, seed, sigma=0.02):
    bits = wl.moe_expert_bits(N, K, E, sigma, 70 + seed, 0)
    qs = [O.quantize(bits[e]) for e in range(E)]
    return (np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]),
            np.array([q[2] for q in qs], dtype=np.float32))


def upload(w):
    return dev_u8(w[0]), dev_u8(w[1]), torch.from_numpy(w[2]).to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    return wl.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def check_grouped(x_bits, row_div, ids, w, got, valid=None, label=""):
    E = w[0].shape[0]
    y64, wn, sa = MO.grouped_gemm_ref(x_bits, row_div, np.where((ids < 0) | (ids >= E), 0, ids), *w)
    K = x_bits.shape[1]
    loose, tight = MO.gemm_bound(x_bits, row_div, y64, wn, sa, K)
    # experts with few pairs run the x-resident decode kernel, which stores each
    # activation row as f16 scaled by a power of two: values below 2^-28 of the
    # row's largest move by at most 2^-39 of it (or 2^-151)
    xf = np.abs(wl.bf16_bits_to_f32(x_bits).astype(np.float64))
    xmax = xf.max(axis=1)[np.arange(y64.shape[0]) // row_div]
    tight = tight + (2.0 ** -39 * xmax[:, None] + 2.0 ** -151) * np.sqrt(K) * wn
    g = f64(got)
    if valid is not None:
        assert np.all(g[~valid] == 0), f"{label}: rows of invalid pairs are not zero"
        g, y64, loose, tight = g[valid], y64[valid], loose[valid], tight[valid]
    err = np.abs(g - y64)
    assert np.all(err <= tight), f"{label}: tight bound, worst {np.max(err - tight):.3e}"
    assert np.all(err <= loose), f"{label}: norm bound"


@pytest.mark.parametrize("E,H,N,T,topk", [
    (8, 512, 512, 5, 2),        # decode-sized: 10 pairs over 8 experts (some empty)
    (4, 1024, 320, 40, 4),      # ~40 pairs per expert: several 16-row tiles, ragged N
    (2, 256, 272, 100, 2),      # 100 pairs per expert: two 64-pair blocks
    (3, 272, 48, 7, 3),         # K % 32 == 16 (8-byte code loads), partial chunk, N < 64
    (5, 48, 300, 9, 1),         # K = 48: one partial chunk
    (2, 768, 256, 30, 2),       # K % 512 != 0: experts with 17..48 pairs take the split-K kernel
    (8, 1024, 4096, 16, 2),     # 8 x 256 tiles fill every wavefront slot (no K split), K % 1024 == 0: the
                                # x-resident kernel's two-region pipeline
])
def test_grouped_gemm_first_layer(E, H, N, T, topk):
    w = experts(E, N, H, E * 100 + N)
    x = wl.random_activation_bits(T, H, seed=T)
    ids, _ = wl.moe_routing(T, E, topk, E + T)
    inv = torch.zeros((), dtype=torch.int32, device=DEV)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), topk, *upload(w), invalid_pairs=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 0
    check_grouped(x, topk, ids.reshape(-1), w, y, label=f"E{E} H{H} N{N} T{T} k{topk}")


def test_grouped_gemm_second_layer_reads_one_row_per_pair():
    E, I, H, P = 6, 256, 520, 37
    w = experts(E, H, I, 11)
    a = wl.random_activation_bits(P, I, seed=12)
    ids = np.random.default_rng(13).integers(0, E, size=P).astype(np.int32)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(a), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(a, 1, ids, w, y, label="second layer")


@pytest.mark.parametrize("K,T", [(256, 6), (1024, 6), (272, 6), (1024, 40)])
def test_invalid_ids_give_zero_rows_and_are_counted(K, T):
    """K = 256 and 1024 with 6 tokens: the x-resident kernel writes the zero
    rows (no split-K launch); K = 272: the split-K kernel does; 40 tokens (20
    pairs per expert on average): the panel kernel takes every expert and
    writes them."""
    E, N, topk = 4, 260, 2
    w = experts(E, N, K, 21)
    x = wl.random_activation_bits(T, K, seed=22)
    ids, _ = wl.moe_routing(T, E, topk, 23)
    ids = ids.reshape(-1).copy()
    ids[3], ids[8] = E, -1
    inv = torch.zeros((), dtype=torch.int32, device=DEV)
    out = torch.full((T * topk, N), 7.0, dtype=torch.bfloat16, device=DEV)
    B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), topk, *upload(w), out=out,
                           invalid_pairs=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 2
    valid = (ids >= 0) & (ids < E)
    check_grouped(x, topk, ids, w, out, valid=valid, label="invalid ids")


def test_all_pairs_on_one_expert_many_blocks():
    E, K, N, T, topk = 3, 512, 256, 150, 1
    w = experts(E, N, K, 31)
    x = wl.random_activation_bits(T, K, seed=32)
    ids = np.full((T, topk), 1, np.int32)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), topk, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, topk, ids.reshape(-1), w, y, label="one expert")


def test_expert_classes_in_one_call():
    """One call mixes experts with few pairs (x-resident kernel), up to 48
    (split-K kernel), more (the blocked kernel) and none."""
    E, K, N = 4, 512, 300
    w = experts(E, N, K, 91)
    counts = {0: 3, 1: 20, 2: 60, 3: 0}
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in counts.items()])
    ids = ids[np.random.default_rng(92).permutation(ids.size)]
    x = wl.random_activation_bits(ids.size, K, seed=93)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, 1, ids, w, y, label="mixed classes")


@pytest.mark.parametrize("counts,N", [((40, 10, 12, 8, 14, 0, 20, 16), 300),
                                      ((70, 6, 6, 6, 6, 6, 6, 6), 300),
                                      ((40, 10, 12, 8, 14, 0, 20, 16), 16400)])
def test_panel_passes_for_experts_beyond_32_pairs(counts, N):
    """At most 16 pairs per active expert on average: one launch of the
    32-row panel kernel takes every expert, those with more than 32 pairs in
    passes of 32 rows over their weights (2 and 3 passes here)."""
    E, K = len(counts), 512
    w = experts(E, N, K, 101 + N)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    ids = ids[np.random.default_rng(102).permutation(ids.size)]
    x = wl.random_activation_bits(ids.size, K, seed=103)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, 1, ids, w, y, label=f"panel passes {counts[0]}")


def test_wide_experts_take_the_512_row_panel_blocks():
    """N >= 16384: experts with 17..64 pairs run the panel kernel with 512-row blocks."""
    E, K, N = 2, 512, 16400
    w = experts(E, N, K, 96)
    ids = np.array([0] * 20 + [1] * 40, np.int32)
    x = wl.random_activation_bits(ids.size, K, seed=97)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, 1, ids, w, y, label="wide experts")


@pytest.mark.parametrize("K,N,E", [(2048, 100, 3), (4096, 300, 2), (8192, 40, 2), (14336, 4096, 8)])
def test_few_tiles_split_k_between_wavefronts(K, N, E):
    """Experts with few rows (few 16-row tiles) and few pairs: the x-resident
    kernel splits each tile's K between 2, 4 or 8 wavefronts (8 at K = 8192
    and 14336, the second layer of one token) and sums their partial tiles;
    tile rounds include slots past the last tile."""
    w = experts(E, N, K, 98 + K)
    ids = (np.arange(3 * E) % E).astype(np.int32)
    x = wl.random_activation_bits(ids.size, K, seed=99)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, 1, ids, w, y, label=f"split K {K}")


def test_long_rows_cap_the_resident_rows():
    """K = 8192: fewer than 12 activation rows fit in LDS, so an expert with
    12 pairs takes the panel kernel while one with 5 stays x-resident."""
    E, K, N = 2, 8192, 80
    w = experts(E, N, K, 94)
    ids = np.array([0] * 5 + [1] * 12, np.int32)
    x = wl.random_activation_bits(ids.size, K, seed=95)
    y = B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w))
    torch.cuda.synchronize()
    check_grouped(x, 1, ids, w, y, label="K 8192")


def test_more_experts_than_routing_threads():
    """E = 1500 > 1024: the routing kernel walks the groups 1024 at a time."""
    E, K, N, P = 1500, 256, 32, 300
    bits = wl.moe_expert_bits(N, K, E, 0.02, 60, 0)
    qs = [O.quantize(bits[e]) for e in range(E)]
    w = (np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]), np.array([q[2] for q in qs], np.float32))
    ids = np.random.default_rng(61).integers(0, E, size=P).astype(np.int32)
    ids[:40] = 7                                           # one expert with many pairs
    ids[40] = E + 3                                        # one id outside [0, E)
    x = wl.random_activation_bits(P, K, seed=62)
    inv = torch.zeros((), dtype=torch.int32, device=DEV)
    out = torch.full((P, N), 5.0, dtype=torch.bfloat16, device=DEV)
    B.nvfp4_moe_w4a16_gemm(dev_bf16(x), torch.from_numpy(ids).to(DEV), 1, *upload(w), out=out, invalid_pairs=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 1
    check_grouped(x, 1, ids, w, out, valid=(ids >= 0) & (ids < E), label="E 1500")


@pytest.mark.parametrize("P,I", [(1, 8), (13, 256), (64, 1000)])
def test_silu_and_mul(P, I):
    rng = np.random.default_rng(P + I)
    h = wl.f32_to_bf16_bits((rng.standard_normal((P, 2 * I)) * 3).astype(np.float32))
    h[0, :4] = wl.f32_to_bf16_bits(np.array([0.0, -0.0, 100.0, -100.0], np.float32))
    a = B.nvfp4_moe_silu_and_mul(dev_bf16(h))
    torch.cuda.synchronize()
    ref = MO.silu_and_mul_ref(h)
    err = np.abs(f64(a) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -133)


@pytest.mark.parametrize("T,topk,H", [(1, 1, 8), (7, 2, 264), (33, 8, 1024)])
def test_combine(T, topk, H):
    rng = np.random.default_rng(T * topk + H)
    o = wl.f32_to_bf16_bits(rng.standard_normal((T * topk, H)).astype(np.float32))
    _, w = wl.moe_routing(T, 16, topk, H)
    out = B.nvfp4_moe_combine(dev_bf16(o), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    ref = MO.combine_ref(o, w)
    sabs = MO.combine_ref(np.bitwise_and(o, 0x7FFF), np.abs(w))
    err = np.abs(f64(out) - ref)
    assert np.all(err <= (topk + 2) * 2.0 ** -24 * sabs + 2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("E,H,I,T,topk", [(8, 512, 256, 5, 2), (4, 256, 384, 30, 3), (3, 272, 48, 4, 2)])
def test_forward_whole_layer(E, H, I, T, topk):
    w13 = experts(E, 2 * I, H, 41 + E)
    w2 = experts(E, H, I, 51 + E)
    x = wl.random_activation_bits(T, H, seed=61 + T)
    ids, tw = wl.moe_routing(T, E, topk, 71 + T)
    inv = torch.zeros((), dtype=torch.int32, device=DEV)
    out = B.nvfp4_moe_w4a16_forward(dev_bf16(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                    upload(w13), upload(w2), invalid_pairs=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 0
    ref = MO.moe_ref(x, ids, tw, w13, w2)
    tol = MO.moe_tolerance(ref, tw, H)
    err = np.abs(f64(out) - ref["out"])
    assert np.all(err <= tol), f"worst excess {np.max(err - tol):.3e}"


def test_forward_empty_batch_enqueues_nothing():
    E, H, I = 2, 64, 32
    w13 = upload(experts(E, 2 * I, H, 81))
    w2 = upload(experts(E, H, I, 82))
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    out = B.nvfp4_moe_w4a16_forward(x, torch.empty((0, 2), dtype=torch.int32, device=DEV),
                                    torch.empty((0, 2), dtype=torch.float32, device=DEV), w13, w2)
    assert out.shape == (0, H)
