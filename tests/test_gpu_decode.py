"""GPU parity of dequant_decode: bit-exact against the oracle's unpack.

Covers every packed byte at every E8M0 exponent (the normative range 2..252
plus the wrapping ends), the MXFP4 GEMV workload's decode sweep (exponents
100..150), the zero bytes at all 256 exponents, a block mixing zero and
non-zero codes, random matrices with a ragged row count, determinism, empty
inputs, and a matrix of more than 2^31 elements (64-bit indexing). Outputs are poisoned before each launch so an unwritten element
cannot pass.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from conftest import golden_ints
from gpu_util import bits, say, u8

pytestmark = pytest.mark.gpu


def run_decode(g, packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    rows, half = packed.shape
    out = torch.full((rows, 2 * half), -1, dtype=torch.int16, device="cuda:0")   # 0xFFFF poison
    g.dequant_decode(u8(packed), u8(scales), out=out)
    return bits(out)


def test_every_byte_at_every_exponent(gpu, orc):
    say("decode: 256 bytes x 256 exponents")
    exps = np.arange(256, dtype=np.uint8)
    packed = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(exps[:, None], 16, axis=1).astype(np.uint8)
    got = run_decode(gpu, packed, scales)
    want = orc.mxfp4_decode(packed, scales)
    normative = slice(2, 253)
    assert np.array_equal(got[normative], want[normative])
    # outside 2..252 both sides follow the integer add; checked for conformance
    assert np.array_equal(got, want)


def test_workload_decode_sweep(gpu, orc):
    say("decode: all bytes x E8M0 100..150")
    packed, scales = synth.decode_sweep_all_bytes(100, 150)
    assert np.array_equal(run_decode(gpu, packed, scales), orc.mxfp4_decode(packed, scales))


def test_zero_codes_at_all_exponents(gpu, orc):
    say("decode: zero bytes x 256 exponents")
    packed, scales = synth.decode_sweep_zero_bytes()
    got = run_decode(gpu, packed, scales)
    assert (got == golden_ints("mxfp4_zero_codes.txt", "expected_bf16")[0]).all()
    assert np.array_equal(got, orc.mxfp4_decode(packed, scales))


def test_zero_and_nonzero_codes_in_one_block(gpu, orc):
    say("decode: mixed block")
    row = np.array([0x00, 0x7A, 0x88, 0x13, 0x08, 0xF1, 0x80, 0x5C] * 2, dtype=np.uint8)
    exps = golden_ints("mxfp4_zero_codes.txt", "mixed_block_e8m0")
    packed = np.tile(row, (len(exps), 1))
    scales = np.array(exps, dtype=np.uint8)[:, None]
    assert np.array_equal(run_decode(gpu, packed, scales), orc.mxfp4_decode(packed, scales))


@pytest.mark.parametrize("rows,k", [(1, 32), (37, 512), (1000, 4096 + 32 * 7), (3, 14336)])
def test_random_matrices(gpu, orc, rows, k):
    say(f"decode: random rows={rows} k={k}")
    r = np.random.default_rng(rows * 7 + k)
    packed = synth.uniform_bytes(r, (rows, k // 2))
    scales = synth.uniform_bytes(r, (rows, k // 32))
    got = run_decode(gpu, packed, scales)
    assert np.array_equal(got, orc.mxfp4_decode(packed, scales))


def test_deterministic_and_empty(gpu):
    say("decode: determinism, empty")
    r = np.random.default_rng(1)
    packed = synth.uniform_bytes(r, (64, 256))
    scales = synth.byte_range(r, (64, 16), 120, 134)
    a = run_decode(gpu, packed, scales)
    b = run_decode(gpu, packed, scales)
    assert np.array_equal(a, b)
    empty = gpu.dequant_decode(u8(np.zeros((0, 16), np.uint8)), u8(np.zeros((0, 1), np.uint8)))
    assert empty.shape == (0, 32)


@pytest.mark.slow
def test_more_than_2_pow_31_elements(gpu, orc):
    """65537 x 32768 codes: 2^31 + 32768 elements, a 4 GiB output, so every index is past the
    32-bit range at the end. Rows at the start, on both sides of element 2^31 (row 65536 starts
    there) and the last row are compared bit for bit; the output is poisoned first."""
    rows, k = 65537, 32768
    r = np.random.default_rng(synth.SEED_BASE + 73)
    packed = r.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = r.integers(100, 151, (rows, k // 32), dtype=np.uint8)
    say(f"decode: {rows} x {k} ({rows * k} elements)")
    out = torch.full((rows, k), -1, dtype=torch.int16, device="cuda:0")
    gpu.dequant_decode(u8(packed), u8(scales), out=out)
    sel = [0, 1, 65534, 65535, 65536]
    got = bits(out[sel])
    want = orc.mxfp4_decode(packed[sel], scales[sel])
    assert np.array_equal(got, want)
