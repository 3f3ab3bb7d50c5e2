"""GPU parity of dequant_gemv_grouped: independent batch-1 MXFP4 products in shared launches.

Each output is compared with the oracle (rel-L2 <= 1e-3 after rounding the fp64
result to the output dtype). Where a matrix's K puts it on the same tile as a
standalone dequant_gemv call (32 < K/32 <= 512), the grouped result must be
bit-identical to that call: the tiles and their summation order are the same.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16, bf16_values, bits, host_f32, rel_l2, say, u8

pytestmark = pytest.mark.gpu

TOL = 1e-3


def run_group(g, orc, cases, out_dtype):
    mats = [(u8(c["packed"]), u8(c["scales"]), bf16(c["x"][0])) for c in cases]
    outs = [torch.full((c["packed"].shape[0],), float("nan"), dtype=out_dtype, device="cuda:0") for c in cases]
    g.dequant_gemv_grouped(mats, out_dtype=out_dtype, outs=outs)
    torch.cuda.synchronize()
    for c, (packed, scales, x), out in zip(cases, mats, outs):
        n, k = c["packed"].shape[0], 2 * c["packed"].shape[1]
        say(f"gemv_grouped: n={n} k={k} out={out_dtype}")
        tag = "f32" if out_dtype == torch.float32 else "bf16"
        want = orc.mxfp4_gemv(c["packed"], c["scales"], c["x"], tag)[0]
        if out_dtype == torch.float32:
            got, want = host_f32(out).astype(np.float64), want.astype(np.float64)
        else:
            got, want = bf16_values(bits(out)), bf16_values(want)
        assert np.isfinite(got).all()
        assert rel_l2(got, want) <= TOL
        if 32 < k // 32 <= 512:
            alone = g.dequant_gemv(packed, scales, x, out_dtype=out_dtype)
            assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                               alone.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    return outs


# (n, k): one-wave tiles of one and two chunks per lane (K <= 2048 / 4096),
# 16-row tiles of seven waves (K = 14336) and of four waves (K = 8192, a
# second launch), K past the grouped kernels (alone), short K (8 lanes per row)
MIXED = [(4099, 4096), (1001, 14336), (45, 1056), (77, 8192), (300, 32 * (64 * 6 + 5)),
         (20, 32768 + 32), (5, 96), (129, 2048)]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mixed_shapes(gpu, orc, out_dtype):
    cases = [synth.mxfp4_gemv_case(synth.SEED_BASE + 90 + i, n, k, 1) for i, (n, k) in enumerate(MIXED)]
    run_group(gpu, orc, cases, out_dtype)


def test_more_matrices_than_one_launch_holds(gpu, orc):
    """Eleven matrices of one tile kind: two launches of up to eight."""
    cases = [synth.mxfp4_gemv_case(synth.SEED_BASE + 110 + i, 33 + 97 * i, 4096 if i % 2 else 14336, 1)
             for i in range(11)]
    run_group(gpu, orc, cases, torch.bfloat16)


def test_llama8b_mlp_shapes_in_one_launch(gpu, orc):
    """Both MLP shapes at batch 1, the full outputs, as the benchmark's grouped step launches them."""
    run_group(gpu, orc, list(synth.llama_mlp_case(synth.SEED_BASE + 3, 1)), torch.bfloat16)


def test_empty_and_zero_k(gpu):
    """n = 0 entries are skipped, k = 0 outputs are zeros, and the others still run."""
    r = np.random.default_rng(synth.SEED_BASE + 130)
    c = synth.mxfp4_gemv_case(synth.SEED_BASE + 131, 64, 4096, 1)
    empty = torch.zeros((0, 2048), dtype=torch.uint8, device="cuda:0")
    mats = [(u8(c["packed"]), u8(c["scales"]), bf16(c["x"][0])),
            (empty, torch.zeros((0, 128), dtype=torch.uint8, device="cuda:0"),
             bf16(synth.bf16_normal(r, (4096,)))),
            (torch.zeros((9, 0), dtype=torch.uint8, device="cuda:0"),
             torch.zeros((9, 0), dtype=torch.uint8, device="cuda:0"),
             torch.zeros((0,), dtype=torch.bfloat16, device="cuda:0"))]
    outs = [torch.full((64,), float("nan"), device="cuda:0"), torch.empty((0,), device="cuda:0"),
            torch.full((9,), float("nan"), device="cuda:0")]
    gpu.dequant_gemv_grouped(mats, outs=outs)
    alone = gpu.dequant_gemv(*mats[0])
    assert torch.equal(outs[0], alone)
    assert torch.equal(outs[2], torch.zeros(9, device="cuda:0"))
    assert gpu.dequant_gemv_grouped([]) == []


def test_graph_replays_match_eager(gpu):
    """The grouped call captured into a HIP graph: every replay equals the eager result."""
    cases = [synth.mxfp4_gemv_case(synth.SEED_BASE + 140 + i, n, k, 1)
             for i, (n, k) in enumerate([(4099, 4096), (1001, 14336), (77, 8192)])]
    mats = [(u8(c["packed"]), u8(c["scales"]), bf16(c["x"][0])) for c in cases]
    eager = [o.clone() for o in gpu.dequant_gemv_grouped(mats, out_dtype=torch.bfloat16)]
    outs = [torch.empty_like(o) for o in eager]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        gpu.dequant_gemv_grouped(mats, out_dtype=torch.bfloat16, outs=outs, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.dequant_gemv_grouped(mats, out_dtype=torch.bfloat16, outs=outs,
                                 stream=torch.cuda.current_stream())
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), rep
