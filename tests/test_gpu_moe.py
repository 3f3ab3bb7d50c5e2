"""GPU parity of mxfp4_moe_gemm against the oracle (rel-L2 <= 1e-2, bf16 output).

The GPU path rounds the activation to bf16 between the two products (the
MFMA operand type); the oracle keeps fp64 throughout and rounds only the
output, so the tolerance absorbs that rounding. Covers the 32-expert, 2880 /
2880, 256-token top-4 layer (every output), ragged extents (column steps that
end mid-way, experts with more tokens than one pass, experts with none),
the page's zero-code invariant, ids outside the expert range, determinism,
and both ways the kernels read the E8M0 scales: staged in LDS per workgroup
(the default) and loaded per step (hidden above 3072 for W13, inter above
3072 for W2, or scale arrays not 16-byte aligned).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from conftest import golden_ints
from gpu_util import bf16, bf16_values, bits, f32, i32, rel_l2, say, u8

pytestmark = pytest.mark.gpu

TOL = 1e-2


def run_moe(g, c):
    out = torch.full(c["x"].shape, -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    g.mxfp4_moe_gemm(bf16(c["x"]), u8(c["w13"]), u8(c["w13_scale"]), u8(c["w2"]), u8(c["w2_scale"]),
                     i32(c["topk_ids"]), f32(c["topk_weights"]), out=out)
    return bits(out)


def check(g, orc, c, tol=TOL):
    T, H = c["x"].shape
    E, two_i, _ = c["w13"].shape
    say(f"moe: T={T} H={H} I={two_i // 2} E={E} topk={c['topk_ids'].shape[1]}")
    got = bf16_values(run_moe(g, c))
    want = bf16_values(orc.mxfp4_moe(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"],
                                     c["topk_ids"], c["topk_weights"]))
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    assert err <= tol, err
    return err


@pytest.mark.slow
def test_workload_32_experts(gpu, orc):
    err = check(gpu, orc, synth.moe_case())
    print(f"rel-L2 {err:.3e}")


@pytest.mark.parametrize("E,H,I,T,topk", [
    (3, 64, 96, 5, 2),          # tiny; one column step
    (4, 160, 224, 33, 2),       # column steps end mid-way (160 = 128 + 32), 224 j's in two blocks
    (2, 288, 64, 100, 2),       # ~100 rows per expert: two token passes
    (8, 2880, 2880, 16, 4),     # the layer's extents with few tokens: some experts get none
    (1, 32, 32, 1, 1),
    (512, 64, 96, 300, 4),      # the most experts the entry point accepts, ~2 pairs each
    (8, 64, 96, 1100, 4),       # 4400 pairs: routing ranks of the fifth 1024-pair chunk go through memory
    (2, 256, 1024, 40, 2),      # W2 rows of 512 bytes: four steps, every row on a 128-byte line
    (1, 64, 1056, 20, 1),       # W2 rows of 528 bytes: line offsets in steps of 16 bytes (period 8), five steps
    (8, 64, 96, 40, 6),         # top-6: the combine's second group of slots is partly empty
])
def test_shapes(gpu, orc, E, H, I, T, topk):
    check(gpu, orc, synth.moe_case(E * 1000 + H + I + T, E, H, I, T, topk))


@pytest.mark.parametrize("E,H,I,T,topk", [
    (2, 3104, 64, 40, 2),       # W13's scale rows too long to stage: per-step scales in the first product
    (1, 64, 3104, 9, 1),        # W2's scale rows too long to stage: per-step scales in the second product
])
def test_scales_loaded_per_step(gpu, orc, E, H, I, T, topk):
    check(gpu, orc, synth.moe_case(E * 1000 + H + I + T, E, H, I, T, topk))


def _unaligned(a: np.ndarray) -> torch.Tensor:
    # a contiguous device copy whose data starts one byte past a 16-byte boundary
    flat = torch.zeros(a.size + 16, dtype=torch.uint8, device="cuda:0")
    v = flat[1:1 + a.size]
    v.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8).ravel()))
    assert v.data_ptr() % 16 == 1
    return v.view(a.shape)


def test_unaligned_scales_take_the_per_step_path(gpu, orc):
    """Scale arrays off a 16-byte boundary are read per step; the result is bit-identical
    to the staged one (same products, same order) and matches the oracle."""
    c = synth.moe_case(31, 4, 160, 224, 33, 2)
    say("moe: unaligned scale arrays")
    staged = run_moe(gpu, c)
    out = torch.full(c["x"].shape, -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    gpu.mxfp4_moe_gemm(bf16(c["x"]), u8(c["w13"]), _unaligned(c["w13_scale"]), u8(c["w2"]),
                       _unaligned(c["w2_scale"]), i32(c["topk_ids"]), f32(c["topk_weights"]), out=out)
    per_step = bits(out)
    assert np.array_equal(per_step, staged)
    want = bf16_values(orc.mxfp4_moe(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"],
                                     c["topk_ids"], c["topk_weights"]))
    assert rel_l2(bf16_values(per_step), want) <= TOL


@pytest.mark.slow
def test_largest_expert(gpu, orc):
    """hidden 32768, inter 65504: one expert's W13 (inter * hidden bytes) just under the 2 GiB
    the entry point accepts, so the weight offsets of the first product reach the top of their
    32-bit range; its scale rows are too long to stage (per-step scale loads)."""
    check(gpu, orc, synth.moe_case(91, 1, 32768, 65504, 2, 1))


def test_every_token_to_the_same_two_experts(gpu, orc):
    """Skewed routing: experts 2 and 5 take every pair, 300 each (five token passes of up to
    64 rows, the last one ragged), the other six experts none."""
    c = synth.moe_case(77, 8, 160, 96, 300, 2)
    ids = np.empty_like(c["topk_ids"])
    ids[:, 0], ids[:, 1] = 2, 5
    c["topk_ids"] = ids
    check(gpu, orc, c)


def test_zero_first_layer_gives_exact_zero(gpu):
    N, K, E, M = golden_ints("mxfp4_zero_codes.txt", "moe_test_shape_N_K_E_M")
    say("moe: zero-code first layer")
    r = np.random.default_rng(0)
    x = synth.bf16_normal(r, (M, K))
    w2, w2s = synth.mxfp4_matrix(r, E * K, N)
    for zb in golden_ints("mxfp4_zero_codes.txt", "zero_bytes"):
        for e in golden_ints("mxfp4_zero_codes.txt", "e8m0_values"):
            c = {"x": x, "w13": np.full((E, 2 * N, K // 2), zb, np.uint8),
                 "w13_scale": np.full((E, 2 * N, K // 32), e, np.uint8),
                 "w2": w2.reshape(E, K, N // 2), "w2_scale": w2s.reshape(E, K, N // 32),
                 "topk_ids": np.zeros((M, 1), np.int32), "topk_weights": np.ones((M, 1), np.float32)}
            assert (run_moe(gpu, c) == 0).all(), (zb, e)


def test_out_of_range_ids_are_skipped(gpu, orc):
    c = synth.moe_case(9, 4, 64, 64, 6, 2)
    ids = c["topk_ids"].copy()
    ids[1, 0], ids[4, 1] = -1, 4
    c_gpu = dict(c, topk_ids=ids)
    say("moe: out-of-range ids")
    got = bf16_values(run_moe(gpu, c_gpu))
    # the same layer with those slots given weight 0 (and a valid id) in the oracle
    ids_o, w_o = ids.copy(), c["topk_weights"].copy()
    bad = (ids_o < 0) | (ids_o >= 4)
    ids_o[bad], w_o[bad] = 0, 0.0
    want = bf16_values(orc.mxfp4_moe(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids_o, w_o))
    assert rel_l2(got, want) <= TOL


def test_deterministic(gpu):
    say("moe: determinism")
    c = synth.moe_case(3, 8, 256, 192, 40, 4)
    assert np.array_equal(run_moe(gpu, c), run_moe(gpu, c))


def test_empty(gpu):
    say("moe: no tokens")
    c = synth.moe_case(3, 2, 64, 64, 1, 1)
    out = gpu.mxfp4_moe_gemm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0"),
                             u8(c["w13"]), u8(c["w13_scale"]), u8(c["w2"]), u8(c["w2_scale"]),
                             torch.zeros((0, 1), dtype=torch.int32, device="cuda:0"),
                             torch.zeros((0, 1), dtype=torch.float32, device="cuda:0"))
    assert out.shape == (0, 64)
