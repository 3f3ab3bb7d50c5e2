"""Pins of the oracle's N:M structured sparsity: encode, decode and the sparse product.

The sglang-jax wiki page on the N:M gap describes the Sparsifier: per group
of M consecutive values the N positions with the largest mask values are
kept, their values gathered, and the in-group positions packed next_log2(M)
bits each, 32 / bits per 32-bit word, entry i at bit (i mod packing) * bits.
Checked here against a brute-force encoder written in this file from that
description (stable top-N of the mask, then the packing formula), a word
packed by hand, decode as the exact inverse of encode on masks with N ones per
group, the sparse product against numpy's dense matmul of the decoded matrix,
and the rejection of positions outside a group.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth

CONFIGS = [(2, 4), (1, 4), (4, 8), (1, 2), (3, 16), (8, 16), (2, 3), (5, 6)]


def brute_encode(dense, mask, n, m):
    rows, k = dense.shape
    bits = max(1, int(np.ceil(np.log2(m))))
    packing = 32 // bits
    per_row = (k // m) * n
    words = -(-per_row // packing)
    vals = np.zeros((rows, per_row), np.uint16)
    meta = np.zeros((rows, words), np.uint64)
    for r in range(rows):
        e = 0
        for g in range(k // m):
            grp = mask[r, g * m:(g + 1) * m].astype(np.int64)
            top = np.argsort(-grp, kind="stable")[:n]   # largest mask values, ties to the lower position
            for pos in sorted(top.tolist()):
                vals[r, e] = dense[r, g * m + pos]
                meta[r, e // packing] |= np.uint64(pos) << np.uint64((e % packing) * bits)
                e += 1
    return vals, meta.astype(np.uint32)


def test_hand_packed_word(orc):
    """2:4, one row of 16 columns: kept positions 2,3 | 0,2 | 0,2 | 0,3 pack as
    2 + 3*4 + 0*16 + 2*64 + 0*256 + 2*1024 + 0*4096 + 3*16384."""
    mask = np.array([[0, 0, 1, 1, 1, 0, 1, 0, 1, 0, 1, 0, 1, 0, 0, 1]], np.uint8)
    dense = np.arange(1, 17, dtype=np.uint16)[None, :]
    vals, meta = orc.nm_encode(dense, mask, 2, 4)
    assert meta.tolist() == [[2 + 3 * 4 + 2 * 64 + 2 * 1024 + 3 * 16384]]
    assert vals.tolist() == [[3, 4, 5, 7, 9, 11, 13, 16]]


@pytest.mark.parametrize("n,m", CONFIGS)
def test_encode_matches_brute_force(orc, n, m):
    r = np.random.default_rng(n * 100 + m)
    rows, k = 5, m * 37
    dense = r.integers(0, 1 << 16, size=(rows, k)).astype(np.uint16)
    mask = r.integers(0, 4, size=(rows, k)).astype(np.uint8)   # general values: ties exercise the order
    vals, meta = orc.nm_encode(dense, mask, n, m)
    bv, bm = brute_encode(dense, mask, n, m)
    assert np.array_equal(vals, bv) and np.array_equal(meta, bm)


@pytest.mark.parametrize("n,m", CONFIGS)
def test_decode_inverts_encode(orc, n, m):
    c = synth.nm_case(n * 7 + m, n, m, rows=9, k=m * 64)
    vals, meta = orc.nm_encode(c["dense"], c["mask"], n, m)
    dense, mask = orc.nm_decode(vals, meta, m * 64, n, m)
    assert np.array_equal(mask, c["mask"])
    assert np.array_equal(dense, np.where(c["mask"] == 1, c["dense"], 0))


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (3, 16)])
def test_spmm_is_the_dense_product_of_the_decode(orc, n, m):
    k = m * 40
    c = synth.nm_case(n + m, n, m, rows=31, k=k, batch=3)
    vals, meta = orc.nm_encode(c["dense"], c["mask"], n, m)
    y = orc.nm_spmm(vals, meta, c["x"], k, n, m)
    w = orc.f64_from_bf16(np.where(c["mask"] == 1, c["dense"], 0))
    want = orc.f64_from_bf16(c["x"]) @ w.T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)


def test_positions_outside_a_group_are_rejected(orc):
    vals = np.zeros((1, 2), np.uint16)
    meta = np.array([[1 | (7 << 3)]], np.uint32)   # 2:6, 3-bit positions: 1 and 7 (> 5)
    with pytest.raises(ValueError):
        orc.nm_decode(vals, meta, 6, 2, 6)
    with pytest.raises(ValueError):
        orc.nm_spmm(vals, meta, np.zeros((1, 6), np.uint16), 6, 2, 6)
