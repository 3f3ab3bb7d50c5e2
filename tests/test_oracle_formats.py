"""Pins of the oracle's number formats: E2M1 table, bf16 rounding, E4M3 decoding,
and the MXFP4 unpack (lookup + integer exponent add + zero forcing).

Each check compares the oracle with something other than itself: the values
the pages print (tests/golden), torch's own CPU casts, or closed forms worked
out by hand below.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from conftest import golden_floats, golden_ints


def torch_bf16_bits_of_f32(values: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- E2M1 ----

def test_e2m1_table_is_the_pages_table(orc):
    assert orc.e2m1_magnitudes() == golden_floats("e2m1_magnitudes.txt", "magnitudes")


# ----------------------------------------------------------------- bf16 ----

def test_bf16_rounding_matches_torch_on_all_float32_classes(orc):
    r = np.random.default_rng(7)
    # random bit patterns over every exponent (normals, subnormals, inf, nan excluded below)
    bits = r.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # exact ties and near-ties in the dropped 16 bits, both parities of the kept LSB
    base = r.integers(0, 2**16, size=4096, dtype=np.uint64).astype(np.uint32) << 16
    extra = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base | 0x0000,
                            base | 0xFFFF])
    bits = np.concatenate([bits, extra]).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    got = orc.bf16_from_f64(f.astype(np.float64))
    want = torch_bf16_bits_of_f32(f)
    assert np.array_equal(got, want)


def test_bf16_nan_and_signed_zero(orc):
    got = orc.bf16_from_f64(np.array([np.nan, -np.nan, 0.0, -0.0, np.inf, -np.inf]))
    assert [hex(v) for v in got] == ["0x7fc0", "0x7fc0", "0x0", "0x8000", "0x7f80", "0xff80"]


def test_bf16_rounds_float64_once(orc):
    # Worked by hand (bf16 keeps 7 fraction bits; spacing 2^-7 in [1, 2)):
    #   1 + 2^-8 is halfway between 0x3F80 and 0x3F81 -> even -> 0x3F80
    #   1 + 3*2^-8 is halfway between 0x3F81 and 0x3F82 -> even -> 0x3F82
    #   1 + 2^-8 + 2^-30 is just above halfway -> 0x3F81 (rounding through float32
    #   first would land on the tie and give 0x3F80: the oracle must not do that)
    #   (2 - 2^-8) * 2^127 is halfway between the largest finite 0x7F7F and 2^128
    #   -> even -> overflow to +inf
    #   2^-133 is the smallest subnormal 0x0001; 2^-134 is a tie with 0 -> 0
    #   3 * 2^-134 is halfway between 0x0001 and 0x0002 -> even -> 0x0002
    vals = [1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-30, (2 - 2**-8) * 2.0**127,
            2.0**-133, 2.0**-134, 3 * 2.0**-134, -(1 + 2**-8 + 2**-30)]
    got = [int(v) for v in orc.bf16_from_f64(np.array(vals))]
    assert got == [0x3F80, 0x3F82, 0x3F81, 0x7F80, 0x0001, 0x0000, 0x0002, 0xBF81]


def test_f64_from_bf16_is_exact(orc):
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    v = orc.f64_from_bf16(bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (v == t) | (np.isnan(v) & np.isnan(t))
    assert same.all()


# ----------------------------------------------------------------- E4M3 ----

def test_e4m3_decoding_matches_torch_float8_e4m3fn(orc):
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = raw.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_f64(b) for b in range(256)])
    for b in range(256):
        if math.isnan(want[b]):
            assert math.isnan(got[b]), b
        else:
            assert got[b] == want[b], (b, got[b], want[b])
    # closed forms: 0x38 = 1.0, 0x01 = 2^-9 (smallest subnormal), 0x7E = 448 (largest)
    assert got[0x38] == 1.0 and got[0x01] == 2.0**-9 and got[0x7E] == 448.0


# ------------------------------------------------------------ MXFP4 unpack --

def _exact_bf16(value: float) -> int:
    """bf16 bits of a value that bf16 represents exactly (torch cast via float32)."""
    return int(torch_bf16_bits_of_f32(np.array([value], dtype=np.float32))[0])


def test_identity_scale_returns_the_table(orc):
    e_id = golden_ints("mxfp4_zero_codes.txt", "identity_e8m0")[0]
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    for code in range(16):
        m = mags[code & 7]
        want = 0x0000 if m == 0.0 else _exact_bf16(-m if code & 8 else m)
        assert orc.mxfp4_decode_one(code, e_id) == want, code


def test_in_range_exponents_give_the_exact_scaled_value(orc):
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    for e in range(2, 253):
        for code in range(16):
            m = mags[code & 7]
            if m == 0.0:
                want = 0x0000
            else:
                want = _exact_bf16(math.ldexp(-m if code & 8 else m, e - 127))
            assert orc.mxfp4_decode_one(code, e) == want, (code, e)


def test_zero_codes_stay_positive_zero_at_every_exponent(orc):
    zero_bytes = golden_ints("mxfp4_zero_codes.txt", "zero_bytes")
    expected = golden_ints("mxfp4_zero_codes.txt", "expected_bf16")[0]
    for e in range(256):
        packed = np.tile(np.array(zero_bytes, dtype=np.uint8), (1, 8))  # 32 bytes -> 64 columns
        scales = np.full((1, 2), e, dtype=np.uint8)
        out = orc.mxfp4_decode(packed, scales)
        assert (out == expected).all(), e
    for b in zero_bytes:
        for e in golden_ints("mxfp4_zero_codes.txt", "e8m0_values"):
            assert orc.mxfp4_decode_one(b & 15, e) == expected
            assert orc.mxfp4_decode_one(b >> 4, e) == expected


def test_zero_and_nonzero_codes_mixed_in_one_block(orc):
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    # bytes alternate an all-zero byte and a byte of two non-zero codes
    row = np.array([0x00, 0x7A, 0x88, 0x13, 0x08, 0xF1, 0x80, 0x5C] * 2, dtype=np.uint8)[None, :]
    for e in golden_ints("mxfp4_zero_codes.txt", "mixed_block_e8m0"):
        out = orc.mxfp4_decode(row, np.full((1, 1), e, dtype=np.uint8))[0]
        for col in range(32):
            byte = int(row[0, col // 2])
            code = (byte & 15) if col % 2 == 0 else (byte >> 4)
            m = mags[code & 7]
            want = 0 if m == 0 else _exact_bf16(math.ldexp(-m if code & 8 else m, e - 127))
            assert out[col] == want, (e, col)


def test_nibble_order_and_scale_blocks(orc):
    # byte 0x7A: column 0 = code 0xA (-1.0), column 1 = code 0x7 (+6.0)
    row = np.zeros((1, 32), dtype=np.uint8)
    row[0, 0] = 0x7A
    row[0, 16] = 0x7A   # first byte of the second 32-column block
    out = orc.mxfp4_decode(row, np.array([[127, 128]], dtype=np.uint8))[0]
    assert (int(out[0]), int(out[1])) == (0xBF80, 0x40C0)           # -1.0, 6.0
    assert (int(out[32]), int(out[33])) == (0xC000, 0x4140)         # -2.0, 12.0
    assert (out[2:32] == 0).all() and (out[34:] == 0).all()


def test_out_of_range_exponents_follow_the_integer_add(orc):
    # Worked by hand from the rule pattern + (e - 127) * 2^7 mod 2^16:
    #   code 7 (0x40C0, 6.0) at e = 255: 0x40C0 + 0x4000 = 0x80C0 (wraps into the sign)
    #   code 1 (0x3F00, 0.5) at e = 1:   0x3F00 + 0xC100 = 0x0000 (mod 2^16)
    #   code 9 (0xBF00,-0.5) at e = 1:   0xBF00 + 0xC100 = 0x8000
    #   code 2 (0x3F80, 1.0) at e = 0:   0x3F80 + 0xC080 = 0x0000
    assert orc.mxfp4_decode_one(7, 255) == 0x80C0
    assert orc.mxfp4_decode_one(1, 1) == 0x0000
    assert orc.mxfp4_decode_one(9, 1) == 0x8000
    assert orc.mxfp4_decode_one(2, 0) == 0x0000


def test_decode_status_on_ragged_k(orc):
    assert orc.load().or_mxfp4_decode(None, None, None, 1, 48) != 0
