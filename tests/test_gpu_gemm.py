"""GPU parity of dequant_gemm (MXFP4 weight GEMM for many activation rows) against the oracle.

The oracle is the MXFP4 product of the GEMV (fp64 sums of the decoded
weights times bf16 x, for any number of rows), rounded to the output dtype
before comparing; the bar is the GEMV's, rel-L2 <= 1e-3 with fp32
accumulation. Shapes span one and many tiles, ragged tiles in both
directions, K with an odd number of 32-column blocks (a half step of zero
weights, the register form), K % 128 == 64 and K % 128 == 0 (the
direct-to-LDS form's two step widths), both output dtypes, block scales over a wide exponent range, and the
prefill shape of the benchmark (2048 tokens through the Llama-8B MLP
matrices) on sampled rows and columns, and the largest K the entry point
accepts under a full 128-row tile.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16, bf16_values, bits, host_f32, rel_l2, say, u8

pytestmark = pytest.mark.gpu

TOL = 1e-3


def gemm_case(g, orc, packed, scales, x, out_dtype):
    n, m = packed.shape[0], x.shape[0]
    say(f"gemm: m={m} n={n} k={x.shape[1]} out={out_dtype}")
    out = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda:0")
    g.dequant_gemm(u8(packed), u8(scales), bf16(x), out=out)
    if out_dtype == torch.float32:
        got = host_f32(out).astype(np.float64)
        want = orc.mxfp4_gemv(packed, scales, x, "f32").astype(np.float64)
    else:
        got = bf16_values(bits(out))
        want = bf16_values(orc.mxfp4_gemv(packed, scales, x, "bf16"))
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    assert err <= TOL, err
    return err


@pytest.mark.parametrize("m,n,k", [
    (1, 16, 32), (17, 40, 64), (128, 128, 64), (130, 300, 96),   # one tile .. ragged, odd block count
    (256, 512, 1024), (129, 129, 2048 + 32), (300, 1000, 4096), (513, 257, 512),
    (64, 300, 192), (257, 513, 320),   # K % 128 == 64: the direct-to-LDS form's 64-column steps, ragged tiles
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_shapes(gpu, orc, m, n, k, out_dtype):
    c = synth.mxfp4_gemv_case(m * 7 + n + k, n, k, batch=m)
    gemm_case(gpu, orc, c["packed"], c["scales"], c["x"], out_dtype)


@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_prefill_shape_sampled(gpu, orc, n, k):
    """2048 tokens through a full Llama-8B MLP matrix, as the benchmark launches
    it; the oracle computes 96 sampled activation rows x 256 sampled weight rows."""
    say(f"gemm: prefill m=2048 n={n} k={k}")
    r = np.random.default_rng(n + k)
    packed = synth.uniform_bytes(r, (n, k // 2))
    scales = synth.byte_range(r, (n, k // 32), 120, 134)
    x = synth.bf16_normal(r, (2048, k))
    out = torch.empty((2048, n), dtype=torch.bfloat16, device="cuda:0")
    gpu.dequant_gemm(u8(packed), u8(scales), bf16(x), out=out)
    got = bf16_values(bits(out))
    rows = np.sort(r.choice(2048, 96, replace=False))
    cols = np.sort(r.choice(n, 256, replace=False))
    want = bf16_values(orc.mxfp4_gemv(packed[cols], scales[cols], x[rows], "bf16"))
    err = rel_l2(got[np.ix_(rows, cols)], want)
    assert err <= TOL, err


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wide_exponent_range(gpu, orc, out_dtype):
    """E8M0 scales over 100..150 (block values from 2^-27 to 6 * 2^23): the decode's
    scale operand and the fp32 accumulation across blocks of very different size."""
    c = synth.mxfp4_gemv_case(77, 300, 1024, batch=140, e_lo=100, e_hi=150)
    gemm_case(gpu, orc, c["packed"], c["scales"], c["x"], out_dtype)


def test_matches_the_gemv_at_small_batch(gpu, orc):
    """For batch <= 16 the GEMM and the GEMV compute the same product."""
    c = synth.mxfp4_gemv_case(5, 640, 2048, batch=12)
    say("gemm: against dequant_gemv")
    y1 = gpu.dequant_gemm(u8(c["packed"]), u8(c["scales"]), bf16(c["x"]), out_dtype=torch.float32)
    y2 = gpu.dequant_gemv(u8(c["packed"]), u8(c["scales"]), bf16(c["x"]), out_dtype=torch.float32)
    assert rel_l2(host_f32(y1), host_f32(y2)) < 1e-6


def test_empty_and_zero_k(gpu):
    say("gemm: empty, k = 0")
    y = torch.full((3, 5), 7.0, device="cuda:0")
    gpu.dequant_gemm(torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"),
                     torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"),
                     torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda:0"), out=y)
    assert (host_f32(y) == 0).all()
    e = gpu.dequant_gemm(torch.zeros((5, 16), dtype=torch.uint8, device="cuda:0"),
                         torch.zeros((5, 1), dtype=torch.uint8, device="cuda:0"),
                         torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda:0"))
    assert e.shape == (0, 5)


@pytest.mark.slow
@pytest.mark.parametrize("k", [8388576, 8388480])
def test_largest_k(gpu, orc, k):
    """k = E2M1_GEMM_MAX_K (the register form: an odd number of 32-column blocks) and the largest
    multiple of 128 below it (the direct-to-LDS form) under a full 128-row tile: the workgroup's
    x offsets reach 2 * 128 * k bytes, just under 2^31 (its 32-bit byte offsets). Rows 0, 1, 126
    and 127 of x carry data and are checked against the oracle; every other row is zero, so its
    outputs must be exact zeros."""
    m, n = 128, 20
    r = np.random.default_rng(synth.SEED_BASE + 71)
    packed, scales = synth.mxfp4_matrix(r, n, k)
    rows = [0, 1, 126, 127]
    x = np.zeros((m, k), np.uint16)
    x[rows] = synth.bf16_normal(r, (len(rows), k))
    say(f"gemm: largest k = {k}, m = {m}, n = {n}")
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.dequant_gemm(u8(packed), u8(scales), bf16(x), out=out)
    got = host_f32(out).astype(np.float64)
    want = orc.mxfp4_gemv(packed, scales, x[rows], "f32").astype(np.float64)
    assert np.isfinite(got).all()
    assert rel_l2(got[rows], want) <= TOL
    assert (got[np.setdiff1d(np.arange(m), rows)] == 0).all()
