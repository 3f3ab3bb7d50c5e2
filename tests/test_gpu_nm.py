"""GPU parity of nm_spmm (N:M structured-sparse weights times bf16 activations) against the oracle.

Tolerance, derived from the arithmetic: every product of two bf16 values is
exact in fp32, and each output is a sum of per_row = (k/M) N such products in
fp32. Both kernels give each lane a sequential chain over about per_row / 64
entries (the fast one in v_dot2_f32_bf16 steps of two entries, at most two
roundings each), then add the 64 lane totals in six DPP steps, so with
u = 2^-24 the error of an output is at most (per_row / 64 + 8) u sum |w x| (a
bound with two spare steps). A bf16 output adds at most 2^-8 |y|. The test
checks every output element against that bound, with sum |w x| from the
oracle's product of the absolute values.

Covers the five configurations with a compiled kernel (2:4, 1:4, 4:8, 1:2,
8:16) at batch 1..4, configurations that take the generic kernel (3:16, 2:3,
5:6, 1:1, 7:8), batches 5..16, activations at and one span above the
staged-LDS limit for one, two and four rows, rows whose kept count is not a
multiple of 8, position words drawn at random (repeats within a group),
unaligned values, the 4096 x 4096 layer and a 14336 x 4096 MLP layer, bf16 output, empty
extents and determinism.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16, host_f32, say, words

pytestmark = pytest.mark.gpu

FAST = [(2, 4), (1, 4), (4, 8), (1, 2), (8, 16)]
GENERIC = [(3, 16), (2, 3), (5, 6), (1, 1), (7, 8)]


def encode(orc, case):
    return orc.nm_encode(case["dense"], case["mask"], case["n"], case["m"])


def run(g, vals, meta, x, n, m, out_dtype=torch.float32, vals_dev=None):
    batch = x.shape[0]
    rows = vals.shape[0]
    out = torch.full((batch, rows), float("nan"), dtype=out_dtype, device="cuda:0")
    v = bf16(vals) if vals_dev is None else vals_dev
    g.nm_spmm(v, words(meta), bf16(x), n, m, out=out)
    return host_f32(out)


def check(g, orc, case, out_dtype=torch.float32, vals_dev=None, label=""):
    n, m, x = case["n"], case["m"], case["x"]
    batch, k = x.shape
    vals, meta = encode(orc, case)
    rows, per_row = vals.shape
    say(f"nm_spmm {n}:{m}: batch={batch} rows={rows} k={k} out={out_dtype} {label}")
    got = run(g, vals, meta, x, n, m, out_dtype, vals_dev)
    want = orc.nm_spmm(vals, meta, x, k, n, m)
    mag = orc.nm_spmm(vals & 0x7FFF, meta, x & 0x7FFF, k, n, m)
    bound = (per_row / 64 + 8) * 2.0 ** -24 * mag + 1e-30
    if out_dtype == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(want)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(np.isfinite(got))
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), f"worst {worst}: got {got[worst]} want {want[worst]} bound {bound[worst]}"
    return got


@pytest.mark.parametrize("n,m", FAST)
@pytest.mark.parametrize("batch", [1, 2, 3, 4])
def test_compiled_configurations(gpu, orc, n, m, batch):
    check(gpu, orc, synth.nm_case(10 * n + m + 100 * batch, n, m, rows=301, k=1024, batch=batch))


@pytest.mark.parametrize("n,m", GENERIC)
def test_generic_configurations(gpu, orc, n, m):
    check(gpu, orc, synth.nm_case(10 * n + m, n, m, rows=133, k=m * 96, batch=2))


@pytest.mark.parametrize("batch", [5, 8, 16])
def test_larger_batches(gpu, orc, batch):
    check(gpu, orc, synth.nm_case(200 + batch, 2, 4, rows=77, k=2048, batch=batch))


@pytest.mark.parametrize("batch,k_in,k_out", [(1, 29120, 29136), (2, 15408, 15424), (4, 7696, 7712)])
def test_lds_limit(gpu, orc, batch, k_in, k_out):
    """Activations staged in 64 KB of LDS: 16-column spans padded to 18 (one row), 34 (two
    interleaved) or 68 (three or four) bf16. k_in is the largest k that fits, k_out the next span."""
    check(gpu, orc, synth.nm_case(300 + batch, 2, 4, rows=64, k=k_in, batch=batch), label="largest staged k")
    check(gpu, orc, synth.nm_case(310 + batch, 2, 4, rows=64, k=k_out, batch=batch), label="one span more")


@pytest.mark.parametrize("n,m,k", [(2, 4, 36), (1, 2, 6), (4, 8, 8), (8, 16, 16), (1, 4, 4)])
def test_short_rows(gpu, orc, n, m, k):
    """Kept counts that are not a multiple of 8 (or k not a multiple of 8), and rows of one group."""
    check(gpu, orc, synth.nm_case(400 + k, n, m, rows=70, k=k, batch=3))


@pytest.mark.parametrize("n,m,batch", [(2, 4, 1), (4, 8, 3), (8, 16, 2), (3, 16, 5)])
def test_arbitrary_positions(gpu, orc, n, m, batch):
    """Position fields drawn at random, repeats within a group included: the encoder never
    writes these, but the product over the kept entries is still defined (every field is
    below M for M a power of two), and both kernels must follow it."""
    r = np.random.default_rng(900 + 16 * n + m)
    k = m * 128
    rows = 97
    bits_ = 1 if m <= 2 else (m - 1).bit_length()
    packing = 32 // bits_
    per_row = (k // m) * n
    words_ = -(-per_row // packing)
    vals = synth.bf16_normal(r, (rows, per_row), 0.02)
    meta = r.integers(0, 2**32, size=(rows, words_), dtype=np.uint64).astype(np.uint32)
    if packing * bits_ < 32:   # 3-bit positions: the two spare high bits of each word stay clear
        meta &= np.uint32((1 << (packing * bits_)) - 1)
    x = synth.bf16_normal(r, (batch, k))
    say(f"nm_spmm {n}:{m}: arbitrary positions, batch={batch}")
    got = run(gpu, vals, meta, x, n, m).astype(np.float64)
    want = orc.nm_spmm(vals, meta, x, k, n, m)
    mag = orc.nm_spmm(vals & 0x7FFF, meta, x & 0x7FFF, k, n, m)
    assert np.all(np.abs(got - want) <= (per_row / 64 + 8) * 2.0 ** -24 * mag + 1e-30)


def test_unaligned_values(gpu, orc):
    case = synth.nm_case(501, 2, 4, rows=40, k=512, batch=1)
    vals, _ = encode(orc, case)
    flat = torch.zeros(vals.size + 1, dtype=torch.bfloat16, device="cuda:0")
    v = flat[1:].view(vals.shape)
    v.copy_(bf16(vals))
    check(gpu, orc, case, vals_dev=v, label="values offset by 2 bytes")


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_llama_layers(gpu, orc, n, m):
    check(gpu, orc, synth.nm_case(600 + m, n, m, rows=4096, k=4096, batch=1))
    check(gpu, orc, synth.nm_case(610 + m, n, m, rows=14336, k=4096, batch=1), label="MLP up")


@pytest.mark.parametrize("n,m", [(2, 4), (3, 16)])
def test_bf16_output(gpu, orc, n, m):
    check(gpu, orc, synth.nm_case(700 + m, n, m, rows=257, k=m * 64, batch=2), out_dtype=torch.bfloat16)


def test_empty(gpu, orc):
    say("nm_spmm: empty extents")
    x = torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda:0")
    vals = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda:0")
    meta = torch.zeros((5, 0), dtype=torch.int32, device="cuda:0")
    y = torch.full((2, 5), float("nan"), device="cuda:0")
    gpu.nm_spmm(vals, meta, x, 2, 4, out=y)
    assert np.array_equal(host_f32(y), np.zeros((2, 5), np.float32))
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda:0")
    vals = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda:0")
    meta = torch.zeros((0, 2), dtype=torch.int32, device="cuda:0")
    assert gpu.nm_spmm(vals, meta, x, 2, 4).shape == (1, 0)


def test_deterministic(gpu, orc):
    case = synth.nm_case(801, 2, 4, rows=1000, k=4096, batch=2)
    vals, meta = encode(orc, case)
    say("nm_spmm: determinism")
    a = run(gpu, vals, meta, case["x"], 2, 4)
    b = run(gpu, vals, meta, case["x"], 2, 4)
    assert np.array_equal(a, b)
