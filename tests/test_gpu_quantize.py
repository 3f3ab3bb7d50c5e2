"""GPU parity of mxfp4_quantize and nvfp4_quantize against the oracle: bit-exact codes and scales.

The quantized codes are integers decided by floating point, so both sides
take each decision from the same value: MXFP4 scales by a power of two
(exact) and NVFP4 takes the same IEEE fp32 steps (fl32(amax / fl32(6 g)),
fl32(e4m3 * g), fl32(x / eff)) before rounding. Covers every finite bf16
pattern (as block contents, so every element value meets every nearby
exponent), random weights at the Llama-8B MLP shape 14336 x 4096, rows of
very different magnitude, blocks with a single non-zero, a ragged last wave,
the round trip through the library's own decoders, empty extents, and more
than 2^31 elements (sampled rows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import bf16, bits, f32, say, u8

pytestmark = pytest.mark.gpu


def all_finite_bf16() -> np.ndarray:
    """Every bf16 pattern with a finite value, padded with zeros to a multiple of 32."""
    p = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (p & 0x7F80) != 0x7F80
    v = p[finite]
    pad = (-v.size) % 32
    return np.concatenate([v, np.zeros(pad, np.uint16)])


def check_mx(g, orc, x_bits):
    rows, k = x_bits.shape
    say(f"mxfp4_quantize: rows={rows} k={k}")
    codes, scales = g.mxfp4_quantize(bf16(x_bits))
    want_c, want_s = orc.mxfp4_quantize(x_bits)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), want_s)
    assert np.array_equal(codes.cpu().numpy(), want_c)


def check_nv(g, orc, x_bits, gs):
    rows, k = x_bits.shape
    say(f"nvfp4_quantize: rows={rows} k={k} g={gs}")
    codes, bs = g.nvfp4_quantize(bf16(x_bits), f32(np.array([gs], np.float32)))
    want_c, want_b = orc.nvfp4_quantize(x_bits, gs)
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), want_b)
    assert np.array_equal(codes.cpu().numpy(), want_c)


def test_mxfp4_every_bf16_pattern(gpu, orc):
    v = all_finite_bf16()
    check_mx(gpu, orc, v.reshape(-1, 64))
    # the same patterns shifted by half a block, so each meets other block maxima
    check_mx(gpu, orc, np.roll(v, 16).reshape(-1, 32))


# 1e-37 and 1e35 put eff = e4m3(bs) * gs below 2^-125 (tiny blocks: eff subnormal) and above
# 2^125 (saturated blocks), where the kernel takes the IEEE divisions instead of a reciprocal.
@pytest.mark.parametrize("gs", [1.0, 0.01, 1.0 / 6.0, 3e-5, 7.25, 1e-37, 1e35])
def test_nvfp4_every_bf16_pattern(gpu, orc, gs):
    check_nv(gpu, orc, all_finite_bf16().reshape(-1, 64), gs)


def test_llama_shape_random_weights(gpu, orc):
    r = np.random.default_rng(21)
    x = orc.bf16_from_f64(r.standard_normal((14336, 4096)) * 0.02)
    check_mx(gpu, orc, x)
    check_nv(gpu, orc, x, 0.02 * 4 / (6 * 448))


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (7, 16 * 33), (33, 4096 + 32), (129, 160)])
def test_shapes_and_magnitudes(gpu, orc, rows, k):
    r = np.random.default_rng(rows * 1000 + k)
    v = r.standard_normal((rows, k)) * (2.0 ** r.integers(-40, 40, size=(rows, 1)))
    v[:, ::7] = 0.0
    v[0, :16] = 0.0
    v[0, 3] = -1e-30   # a block with a single tiny non-zero
    x = orc.bf16_from_f64(v)
    if k % 32 == 0:
        check_mx(gpu, orc, x)
    check_nv(gpu, orc, x, 0.5)


def test_round_trip_through_the_decoders(gpu, orc):
    """quantize(decode(c, e)) = (c, e) on the GPU for blocks whose largest magnitude is 6."""
    say("quantize: round trip")
    r = np.random.default_rng(22)
    rows, k = 256, 1024
    codes = r.integers(0, 16, size=(rows, k)).astype(np.uint8)
    codes[:, ::32] = 7
    e = r.integers(2, 253, size=(rows, k // 32)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    x = gpu.dequant_decode(u8(packed), u8(e))
    c2, e2 = gpu.mxfp4_quantize(x)
    assert np.array_equal(e2.cpu().numpy(), e)
    got = c2.cpu().numpy()
    want = np.where((codes & 7) == 0, 0, codes)
    assert np.array_equal(got & 15, (want[:, 0::2] | (want[:, 1::2] << 4)) & 15)
    assert np.array_equal(got, (want[:, 0::2] | (want[:, 1::2] << 4)).astype(np.uint8))


def test_empty(gpu):
    say("quantize: empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    c, s = gpu.mxfp4_quantize(x)
    assert c.shape == (0, 32) and s.shape == (0, 2)
    c, s = gpu.nvfp4_quantize(x, torch.ones(1, device="cuda:0"))
    assert c.shape == (0, 32) and s.shape == (0, 4)


@pytest.mark.slow
def test_more_than_2_pow_31_elements(gpu, orc):
    """65537 x 32768 bf16 (2^31 + 32768 elements, 4.3 GB): the element offsets of the last row
    and the code offsets of the last two rows are past the 32-bit range. Rows 0, 1, 65534,
    65535 and 65536 of both quantizers are compared bit for bit with the oracle."""
    rows, k = 65537, 32768
    r = np.random.default_rng(31)
    x = r.integers(0, 1 << 16, (rows, k), dtype=np.uint16)
    np.bitwise_and(x, 0xBFFF, out=x)   # exponent field below 128: every value finite
    sel = np.array([0, 1, rows - 3, rows - 2, rows - 1])
    sel_dev = torch.from_numpy(sel).to("cuda:0")
    say(f"quantize: rows={rows} k={k} ({rows * k} elements)")
    xd = bf16(x)
    codes, scales = gpu.mxfp4_quantize(xd)
    want_c, want_s = orc.mxfp4_quantize(x[sel])
    assert np.array_equal(scales[sel_dev].cpu().numpy(), want_s)
    assert np.array_equal(codes[sel_dev].cpu().numpy(), want_c)
    del codes, scales
    gs = 2.0 / (6 * 448)   # every |x| < 2: the block scales stay inside E4M3
    codes, bs = gpu.nvfp4_quantize(xd, f32(np.array([gs], np.float32)))
    want_c, want_b = orc.nvfp4_quantize(x[sel], gs)
    assert np.array_equal(bs[sel_dev].cpu().numpy(), want_b)
    assert np.array_equal(codes[sel_dev].cpu().numpy(), want_c)
