"""GPU parity of dequant_gemv against the oracle (rel-L2 <= 1e-3, fp32 accumulate).

The oracle's fp64 result is rounded to the output dtype before comparing
(fp32, or bf16 round-to-nearest-even). Shapes span several tiles, ragged row
counts and ragged 32-column chunk counts per lane, every batch size path,
both output dtypes, the Llama-8B MLP shapes at batch 1, 4 and 16 (the full
outputs, exactly as the benchmark launches them), and more than 2 GiB of codes
(sampled rows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from conftest import golden_ints
from gpu_util import bf16, bf16_values, bits, host_f32, rel_l2, say, u8

pytestmark = pytest.mark.gpu

TOL = 1e-3


def gemv_case(g, orc, case, out_dtype):
    say(f"gemv: n={case['packed'].shape[0]} k={2 * case['packed'].shape[1]} "
        f"batch={case['x'].shape[0]} out={out_dtype}")
    n = case["packed"].shape[0]
    batch = case["x"].shape[0]
    out = torch.full((batch, n), float("nan"), dtype=out_dtype, device="cuda:0")
    g.dequant_gemv(u8(case["packed"]), u8(case["scales"]), bf16(case["x"]), out_dtype=out_dtype, out=out)
    if out_dtype == torch.float32:
        got = host_f32(out).astype(np.float64)
        want = orc.mxfp4_gemv(case["packed"], case["scales"], case["x"], "f32").astype(np.float64)
    else:
        got = bf16_values(bits(out))
        want = bf16_values(orc.mxfp4_gemv(case["packed"], case["scales"], case["x"], "bf16"))
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    assert err <= TOL, err
    return err


def test_small_workload_fp32(gpu, orc):
    err = gemv_case(gpu, orc, synth.gemv_small(), torch.float32)
    assert err < 1e-6


SHAPES = [
    (8, 32, 1), (5, 96, 1), (33, 256, 1), (70, 512, 1), (129, 1024, 1),   # 8 to 32 lanes per row
    (45, 1056, 1), (99, 3104, 1),     # one wave per four rows: one and two chunks per lane, ragged
    (4099, 4096, 1),                  # one wave per four rows, ragged last group
    (300, 32 * (64 * 2 + 5), 1),      # row tiles of 16, three waves, the last one ragged
    (257, 4096, 1), (77, 8192, 1),    # four rows per wave; 16-row tiles of four waves
    (64, 8192 + 32, 1),               # five waves, one chunk in the last
    (1001, 14336, 1),                 # seven waves (the down projection's K)
    (40, 16384 + 32 * 3, 1), (50, 32768, 1),   # K-split kernel, 9 and 16 waves
    (20, 32768 + 32, 1),              # beyond the batch-1 kernels -> generic kernel
    (70001, 2048, 1),                 # many row tiles, ragged last one
    (17000, 16384 + 32, 1),           # > 64 rows per workgroup in the K-split kernel
    (31, 512, 2), (17, 4096 + 32, 3), (9, 1024, 4), (65, 2048, 8), (12, 768, 16),
    # batch 2 to 4 in the batch-1 tile layout: two to sixteen waves, ragged chunks and rows
    (47, 1024 + 32, 2), (100, 14336, 2), (33, 16384, 3), (290, 32 * 200 + 32 * 7, 2), (18, 8192, 3),
    (61, 32 * 77, 4), (35, 16384, 4), (129, 4096, 4),
    # batch 5 to 16 on the matrix cores: ragged last slice, rows not a multiple of 8 or 16, the down
    # projection's K; batch 4 at the down projection's K
    (77, 1024 * 3 + 32 * 5, 5), (130, 14336, 4), (1000, 2080, 7), (1003, 4096, 6), (258, 4096, 16),
    (33, 14336, 8), (40, 32 * 40, 16),
    # batch above 1 with K beyond the tiled kernels: one wave per row
    (21, 16384 + 32, 5), (9, 16384 + 64, 2),
]


@pytest.mark.parametrize("n,k,batch", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_shapes(gpu, orc, n, k, batch, out_dtype):
    gemv_case(gpu, orc, synth.mxfp4_gemv_case(n * 31 + k + batch, n, k, batch), out_dtype)


def test_wide_exponent_range(gpu, orc):
    r = np.random.default_rng(77)
    packed, scales = synth.mxfp4_matrix(r, 96, 2048, 100, 154)
    gemv_case(gpu, orc, {"packed": packed, "scales": scales, "x": synth.bf16_normal(r, (1, 2048))},
              torch.float32)


def test_zero_codes_give_exact_zero(gpu):
    say("gemv: zero codes")
    r = np.random.default_rng(3)
    zb = np.array(golden_ints("mxfp4_zero_codes.txt", "zero_bytes"), dtype=np.uint8)
    packed = r.choice(zb, size=(128, 2048))
    scales = r.integers(0, 256, size=(128, 128), dtype=np.uint8)   # every exponent, 255 included
    scales[:, :2] = [0, 255]
    for batch in (1, 4, 16):
        y = gpu.dequant_gemv(u8(packed), u8(scales), bf16(synth.bf16_normal(r, (batch, 4096))))
        assert (host_f32(y) == 0).all()


def test_k_zero_and_n_zero(gpu):
    say("gemv: empty extents")
    y = torch.full((2, 5), 7.0, device="cuda:0")
    gpu.dequant_gemv(u8(np.zeros((5, 0), np.uint8)), u8(np.zeros((5, 0), np.uint8)),
                     torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda:0"), out=y)
    assert (host_f32(y) == 0).all()
    y0 = gpu.dequant_gemv(u8(np.zeros((0, 16), np.uint8)), u8(np.zeros((0, 1), np.uint8)),
                          torch.zeros((1, 32), dtype=torch.bfloat16, device="cuda:0"))
    assert y0.shape == (1, 0)


@pytest.mark.slow
@pytest.mark.parametrize("batch", [1, 4, 16])
def test_llama8b_mlp_shapes(gpu, orc, batch):
    for case in synth.llama_mlp_case(synth.SEED_BASE + 3, batch):
        gemv_case(gpu, orc, case, torch.bfloat16)


def test_deterministic(gpu):
    say("gemv: determinism")
    case = synth.mxfp4_gemv_case(5, 1024, 4096, 1)
    args = (u8(case["packed"]), u8(case["scales"]), bf16(case["x"]))
    a = host_f32(gpu.dequant_gemv(*args))
    b = host_f32(gpu.dequant_gemv(*args))
    assert np.array_equal(a, b)


@pytest.mark.slow
@pytest.mark.parametrize("batch", [1, 4])
def test_more_than_2_gib_of_codes(gpu, orc, batch):
    """140000 x 32768: 2.29 GB of codes, so the byte offsets of the last rows are past the
    32-bit range. The first and last 64 rows of the output are compared with the oracle."""
    n, k = 140000, 32768
    r = np.random.default_rng(synth.SEED_BASE + 74 + batch)
    packed = r.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = r.integers(120, 135, (n, k // 32), dtype=np.uint8)
    x = synth.bf16_normal(r, (batch, k))
    say(f"gemv: n={n} k={k} batch={batch} ({n * k // 2} bytes of codes)")
    out = torch.full((batch, n), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.dequant_gemv(u8(packed), u8(scales), bf16(x), out_dtype=torch.float32, out=out)
    got = host_f32(out).astype(np.float64)
    sel = np.r_[0:64, n - 64:n]
    want = orc.mxfp4_gemv(packed[sel], scales[sel], x, "f32").astype(np.float64)
    assert np.isfinite(got).all()
    assert rel_l2(got[:, sel], want) <= TOL
