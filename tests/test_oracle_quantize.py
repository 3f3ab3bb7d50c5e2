"""Pins of the oracle's MXFP4 and NVFP4 quantizers (the encode side of the formats).

The pages print no encoder: the vLLM page's MoE test calls an MXFP4 quantizer
on bf16 weights and shows only its outputs, the SGLang page only dequantises
NVFP4. The reading taken (OCP microscaling for the MXFP4 block exponent, and
nearest E2M1 value with ties to the even code, saturating at 6, for the
elements) is therefore parity-unpinned in its rounding rule, and pinned here
by what the formats fix: the decoders of the pages are its inverse on every
block they can produce (round trips through the separately pinned decode and
gather), hand-worked values at every tie of the E2M1 grid, the E8M0 exponent
of blocks with known largest elements, torch's float8_e4m3fn cast for the
E4M3 block scale, and the error bound of rounding to nearest.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth

MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [rows, k] (4-bit) -> bytes [rows, k/2], low nibble = even column."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    out = np.empty((packed.shape[0], 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def test_e2m1_ties_and_saturation(orc):
    # midpoints of the grid {0, .5, 1, 1.5, 2, 3, 4, 6} go to the code whose last bit is 0
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (0.2499, 0), (0.2501, 1), (5.0001, 7), (5.9, 7), (6.0, 7), (7.5, 7), (1e30, 7),
             (0.0, 0), (-0.0, 8), (-0.75, 10), (-0.1, 8), (-6.5, 15)]
    for v, code in cases:
        assert orc.e2m1_encode(v) == code, v
    # every grid value maps to its own code
    for i, m in enumerate(MAG):
        assert orc.e2m1_encode(m) == i and orc.e2m1_encode(-m) == (8 | i if m > 0 else 8)


def test_e4m3_encode_matches_torch_cast(orc):
    """Nearest E4M3 value, ties to even, over every representable value, every
    midpoint and random values in [0, 448] (torch's cast rounds the same way)."""
    vals = [orc.e4m3_to_f64(b) for b in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    rnd = np.random.default_rng(7).uniform(0, 448, 4000).tolist()
    tiny = np.random.default_rng(8).uniform(0, 2.0 ** -6, 1000).tolist()
    for t in vals + mids + rnd + tiny:
        t32 = float(np.float32(t))
        want = int(torch.tensor([t32], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item())
        assert orc.e4m3_encode(t32) == want, t32
    assert orc.e4m3_encode(448.0) == 0x7E and orc.e4m3_encode(1e9) == 0x7E


def block_codes(r, rows, k):
    """Random 4-bit codes whose every 32-column block holds a magnitude 4 or 6 code."""
    codes = r.integers(0, 16, size=(rows, k)).astype(np.uint8)
    top = r.choice(np.array([6, 7, 14, 15], dtype=np.uint8), size=(rows, k // 32))
    pos = r.integers(0, 32, size=(rows, k // 32))
    for b in range(k // 32):
        codes[np.arange(rows), 32 * b + pos[:, b]] = top[:, b]
    return codes


def test_mxfp4_round_trip(orc):
    """quantize(decode(c, e)) = (c, e) for every block whose largest magnitude is 4 or
    6, with both zero codes read as code 0 (the decoder maps them to +0)."""
    r = np.random.default_rng(11)
    rows, k = 64, 512
    codes = block_codes(r, rows, k)
    e = r.integers(2, 253, size=(rows, k // 32)).astype(np.uint8)
    x = orc.mxfp4_decode(pack_codes(codes), e)
    packed, scales = orc.mxfp4_quantize(x)
    assert np.array_equal(scales, e)
    want = np.where((codes & 7) == 0, 0, codes)
    assert np.array_equal(unpack_codes(packed), want)


def test_mxfp4_block_exponent(orc):
    """The exponent is floor(log2(amax)) - 2 + 127: blocks whose largest |x| is
    2^j times 1, 1.5 or 1.99 get j + 125; all-zero blocks 0; tiny blocks clamp at 0."""
    rows = []
    want = []
    for j in (-100, -10, -1, 0, 1, 5, 100):
        for f in (1.0, 1.5, 1.99):
            v = np.zeros(32)
            v[7] = -f * 2.0 ** j
            v[3] = 0.3 * 2.0 ** j
            rows.append(v)
            want.append(j + 125)
    rows.append(np.zeros(32))
    want.append(0)
    v = np.zeros(32)
    v[0] = 2.0 ** -130
    rows.append(v)
    want.append(0)
    x = orc.bf16_from_f64(np.array(rows))
    _, scales = orc.mxfp4_quantize(x)
    assert scales[:, 0].tolist() == want


def test_mxfp4_error_bound_on_random_weights(orc):
    """Rounding to nearest: every decoded element within the grid lies within half
    an E2M1 step of its input, the step being that of the grid cell the scaled input
    falls in; scaled inputs above 6 (the block exponent puts the largest in [4, 8))
    decode to 6 units with their sign."""
    r = np.random.default_rng(12)
    x = orc.bf16_from_f64(r.standard_normal((32, 1024)) / 10)
    packed, scales = orc.mxfp4_quantize(x)
    back = orc.f64_from_bf16(orc.mxfp4_decode(packed, scales))
    xv = orc.f64_from_bf16(x)
    unit = 2.0 ** (np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    a = np.abs(xv) / unit
    assert (a < 8).all()
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    inside = a <= 6
    assert (np.abs(back - xv) <= step / 2 * unit)[inside].all()
    assert np.array_equal(back[~inside], np.sign(xv[~inside]) * 6 * unit[~inside])
    assert (~inside).sum() > 0


def test_nvfp4_round_trip(orc):
    """quantize(gather(c, bs, g)) = (c, bs) at the workload's global scale: the
    bf16 rounding of the dequantised values moves them by 2^-9 at most, far inside
    half a step of either grid."""
    r = np.random.default_rng(13)
    rows, k, g = 48, 256, np.float32(0.01)
    codes = r.integers(0, 16, size=(rows, k)).astype(np.uint8)
    top = r.choice(np.array([7, 15], dtype=np.uint8), size=(rows, k // 16))
    pos = r.integers(0, 16, size=(rows, k // 16))
    for b in range(k // 16):
        codes[np.arange(rows), 16 * b + pos[:, b]] = top[:, b]
    bs = r.integers(0x10, 0x70, size=(rows, k // 16)).astype(np.uint8)
    x, bad = orc.nvfp4_gather(pack_codes(codes), bs, g, np.arange(rows))
    assert bad == 0
    packed, bs2 = orc.nvfp4_quantize(x, g)
    assert np.array_equal(bs2, bs)
    want = np.where((codes & 7) == 0, codes & 8, codes)   # +/-0 keep the sign of the bf16 zero
    got = unpack_codes(packed)
    assert np.array_equal(got & 7, want & 7)
    nonzero = (codes & 7) != 0
    assert np.array_equal(got[nonzero], codes[nonzero])


def test_nvfp4_hand_worked(orc):
    """g = 1, block amax 6: scale byte 0x38 (1.0), elements at every tie of the grid."""
    v = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -6.0, 0, 0.5, 1, 1.5, 2, 3])
    packed, bs = orc.nvfp4_quantize(orc.bf16_from_f64(v[None, :]), 1.0)
    assert bs.tolist() == [[0x38]]
    assert unpack_codes(packed)[0].tolist() == [7, 0, 2, 2, 4, 4, 6, 6, 10, 15, 0, 1, 2, 3, 4, 5]


def test_quantizers_reject_what_they_cannot_encode(orc):
    x = orc.bf16_from_f64(np.ones((1, 32)))
    x[0, 5] = 0x7FC0   # NaN
    with pytest.raises(ValueError):
        orc.mxfp4_quantize(x)
    with pytest.raises(ValueError):
        orc.nvfp4_quantize(x, 1.0)
    with pytest.raises(ValueError):
        orc.nvfp4_quantize(orc.bf16_from_f64(np.ones((1, 32))), 0.0)
