"""Pins of the oracle's products: MXFP4 GEMV, ternary GEMV, NVFP4 gather, MXFP4 MoE.

Each check ties the oracle to something outside itself: numpy's dense matmul
of a separately pinned decode, closed-form special cases, the packing rule as
the page states it (applied in the encode direction), torch casts, the page's
own element-loop order, and the page's invariants (zero codes collapse the
MoE layer to exact zeros).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import expit

import synth
from conftest import golden_floats, golden_ints


def dense_mxfp4(orc, packed, scales) -> np.ndarray:
    """Dense float64 weights through the (separately pinned) unpack."""
    return orc.f64_from_bf16(orc.mxfp4_decode(packed, scales))


# -------------------------------------------------------------- MXFP4 GEMV --

@pytest.mark.parametrize("n,k,batch", [(8, 64, 1), (5, 96, 3), (17, 256, 16)])
def test_gemv_is_a_dense_matmul(orc, n, k, batch):
    case = synth.mxfp4_gemv_case(11 + n, n, k, batch)
    w = dense_mxfp4(orc, case["packed"], case["scales"])
    x = orc.f64_from_bf16(case["x"])
    want = x @ w.T
    got = orc.mxfp4_gemv_f64(case["packed"], case["scales"], case["x"])
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_gemv_output_rounding(orc):
    case = synth.mxfp4_gemv_case(5, 64, 128, 2)
    y64 = orc.mxfp4_gemv_f64(case["packed"], case["scales"], case["x"])
    assert np.array_equal(orc.mxfp4_gemv(case["packed"], case["scales"], case["x"], "f32"),
                          y64.astype(np.float32))
    assert np.array_equal(orc.mxfp4_gemv(case["packed"], case["scales"], case["x"], "bf16"),
                          orc.bf16_from_f64(y64))


def test_gemv_all_zero_codes_give_exact_zero(orc):
    zero_bytes = golden_ints("mxfp4_zero_codes.txt", "zero_bytes")
    r = np.random.default_rng(3)
    packed = r.choice(np.array(zero_bytes, dtype=np.uint8), size=(16, 64))
    scales = r.integers(0, 256, size=(16, 4), dtype=np.uint8)
    x = synth.bf16_normal(r, (2, 128))
    y = orc.mxfp4_gemv_f64(packed, scales, x)
    assert (y == 0).all()


def test_gemv_one_hot_weight(orc):
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    r = np.random.default_rng(4)
    x = synth.bf16_normal(r, (1, 64))
    xv = orc.f64_from_bf16(x)[0]
    for col in (0, 1, 30, 33, 63):
        for code in (1, 7, 12):
            packed = np.zeros((1, 32), dtype=np.uint8)
            packed[0, col // 2] = code if col % 2 == 0 else code << 4
            scales = np.array([[127, 129]], dtype=np.uint8)
            y = orc.mxfp4_gemv_f64(packed, scales, x)[0, 0]
            m = mags[code & 7] * (-1 if code & 8 else 1) * (1 if col < 32 else 4)
            assert y == m * xv[col], (col, code)


def test_gemv_exponent_shift_scales_exactly(orc):
    case = synth.mxfp4_gemv_case(9, 12, 128, 1)
    y = orc.mxfp4_gemv_f64(case["packed"], case["scales"], case["x"])
    y2 = orc.mxfp4_gemv_f64(case["packed"], case["scales"] + 3, case["x"])
    assert np.array_equal(y2, 8.0 * y)


# ----------------------------------------------------------------- ternary --

def pack_ternary(t: np.ndarray) -> np.ndarray:
    """Encode {-1, 0, +1} [n, k] with the page's packing formula (encode direction):
    word = sum_k [1(w_k = +1) 2^(2k+1) + 1(w_k = -1) 2^(2k)] over 16 weights."""
    n, k = t.shape
    out = np.zeros((n, k // 16), dtype=np.uint64)
    for j in range(16):
        col = t[:, j::16]
        out += (col == 1).astype(np.uint64) << np.uint64(2 * j + 1)
        out += (col == -1).astype(np.uint64) << np.uint64(2 * j)
    return out.astype(np.uint32)


def test_ternary_masks_match_the_page():
    assert golden_ints("ternary_encoding.txt", "plus_mask")[0] == int(
        pack_ternary(np.ones((1, 16), dtype=np.int64))[0, 0])
    assert golden_ints("ternary_encoding.txt", "minus_mask")[0] == int(
        pack_ternary(-np.ones((1, 16), dtype=np.int64))[0, 0])


def test_ternary_single_weight_at_every_position(orc):
    r = np.random.default_rng(2)
    x = r.standard_normal(32).astype(np.float32)
    s = np.array([0.0625], dtype=np.float32)
    for word in range(2):
        for j in range(16):
            for sign, bit in ((+1, 2 * j + 1), (-1, 2 * j)):
                packed = np.zeros((1, 2), dtype=np.uint32)
                packed[0, word] = np.uint32(1 << bit)
                y = orc.ternary_gemv(packed, s, x)[0]
                want = np.float32(np.float64(s[0]) * sign * np.float64(x[16 * word + j]))
                assert y == want, (word, j, sign)


@pytest.mark.parametrize("n,k", [(7, 16), (9, 160), (33, 512)])
def test_ternary_matches_dense_product(orc, n, k):
    r = np.random.default_rng(n * 1000 + k)
    t = r.integers(-1, 2, size=(n, k))
    x = r.standard_normal(k).astype(np.float32)
    s = r.uniform(0.01, 0.1, size=n).astype(np.float32)
    y, y64 = orc.ternary_gemv(pack_ternary(t), s, x, want_f64=True)
    want = s.astype(np.float64) * (t.astype(np.float64) @ x.astype(np.float64))
    np.testing.assert_allclose(y64, want, rtol=1e-13, atol=1e-15)
    assert np.array_equal(y, y64.astype(np.float32))


def test_ternary_zero_row_and_invalid_pattern(orc):
    x = np.ones(32, dtype=np.float32)
    assert (orc.ternary_gemv(np.zeros((3, 2), dtype=np.uint32), np.ones(3, np.float32), x) == 0).all()
    with pytest.raises(ValueError):
        orc.ternary_gemv(np.array([[0b11, 0]], dtype=np.uint32), np.ones(1, np.float32), x)


def test_ternary_generator_draws_only_the_three_patterns():
    words = synth.two_bit_words(np.random.default_rng(0), 64, 256)
    fields = (words[..., None] >> (2 * np.arange(16, dtype=np.uint32))) & 3
    assert set(np.unique(fields).tolist()) == {0, 1, 2}


# ------------------------------------------------------------------- NVFP4 --

def test_nvfp4_identity_scales_give_the_table(orc):
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    one = 0x38  # E4M3 byte of 1.0
    for code in range(16):
        m = mags[code & 7]
        v = np.float32(-m if code & 8 else m)  # code 8 is -0.0: the sign is kept
        want = int(torch.tensor([v]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert orc.nvfp4_element(code, one, 1.0) == want, code
    assert orc.nvfp4_element(8, one, 1.0) == 0x8000


def test_nvfp4_fp32_order(orc):
    # value * float(scale * global) in fp32, then bf16: check against torch doing
    # the same three steps in float32 on every (scale byte, code) pair.
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    g = np.float32(0.37)
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    bs = raw.view(torch.float8_e4m3fn).to(torch.float32)
    for code in range(16):
        m = mags[code & 7]
        v = torch.tensor(-m if code & 8 else m, dtype=torch.float32)
        eff = bs * torch.tensor(g, dtype=torch.float32)
        want = (v * eff).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        for b in range(256):
            if torch.isnan(bs[b]):
                continue
            assert orc.nvfp4_element(code, b, g) == want[b], (code, b)


def test_nvfp4_page_orders_agree_at_global_scale_0p01(orc):
    # The page's implementation multiplies in float32; its test reference
    # multiplies in Python floats and stores float32. At the workload's global
    # scale the two orders give the same bf16 for every non-NaN scale byte and code.
    mags = golden_floats("e2m1_magnitudes.txt", "magnitudes")
    g = np.float32(0.01)
    mismatches = 0
    for b in range(256):
        s = orc.e4m3_to_f64(b)
        if np.isnan(s):
            continue
        for code in range(16):
            m = mags[code & 7]
            value = -m if code & 8 else m
            f = np.float32(value * (s * float(g)))
            ref = int(torch.tensor([f]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
            mismatches += ref != orc.nvfp4_element(code, b, g)
    assert mismatches == 0


def test_nvfp4_gather_matches_page_element_loop(orc):
    r = np.random.default_rng(12)
    table = synth.uniform_bytes(r, (40, 48))       # hidden 96 = 6 groups
    bscale = synth.e4m3_log2_uniform(r, (40, 6))
    ids = np.array([3, 0, 39, 3, 17], dtype=np.int64)
    got, bad = orc.nvfp4_gather(table, bscale, 0.01, ids)
    assert bad == 0
    loop = orc.nvfp4_gather_elementwise(table, bscale, 0.01, ids)
    want = torch.from_numpy(loop).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_nvfp4_layout_groups_and_row_selection(orc):
    g = golden_ints("nvfp4_layout.txt", "group_size")[0]
    table = np.zeros((3, 16), dtype=np.uint8)      # hidden 32 = 2 groups
    table[2, 0] = 0x7A                              # col 0 low nibble -1.0, col 1 high nibble 6.0
    table[2, g // 2] = 0x7A                         # first byte of group 1
    bscale = np.full((3, 2), 0x38, dtype=np.uint8)  # 1.0
    bscale[2, 1] = 0x40                             # 2.0 for group 1
    out, _ = orc.nvfp4_gather(table, bscale, 1.0, np.array([2, 1]))
    assert (int(out[0, 0]), int(out[0, 1])) == (0xBF80, 0x40C0)
    assert (int(out[0, g]), int(out[0, g + 1])) == (0xC000, 0x4140)
    assert (out[1] == 0).all()


def test_nvfp4_bad_ids_and_guard(orc):
    table = np.full((4, 8), 0x11, dtype=np.uint8)
    bscale = np.full((4, 1), 0x38, dtype=np.uint8)
    out, bad = orc.nvfp4_gather(table, bscale, 1.0, np.array([-1, 4, 1]))
    assert bad == 2 and (out[:2] == 0).all() and (out[2] == 0x3F00).all()
    # hidden must be a multiple of the group size (the page's create_weights guard)
    assert orc.load().or_nvfp4_gather(None, None, 1.0, None, None, 4, 24, 0, None) != 0


# --------------------------------------------------------------------- MoE --

def test_moe_zero_first_layer_collapses_to_zero(orc):
    # the page's test: every W13 byte is a zero code, W2 random, one expert slot
    # with weight 1; silu(0) * 0 = 0, so the layer output is exactly zero.
    N, K, E, M = golden_ints("mxfp4_zero_codes.txt", "moe_test_shape_N_K_E_M")
    r = np.random.default_rng(0)
    x = synth.bf16_normal(r, (M, K))
    w2, w2s = synth.mxfp4_matrix(r, E * K, N)
    ids = np.zeros((M, 1), dtype=np.int32)
    wts = np.ones((M, 1), dtype=np.float32)
    for zb in golden_ints("mxfp4_zero_codes.txt", "zero_bytes"):
        for e in golden_ints("mxfp4_zero_codes.txt", "e8m0_values"):
            w13 = np.full((E, 2 * N, K // 2), zb, dtype=np.uint8)
            w13s = np.full((E, 2 * N, K // 32), e, dtype=np.uint8)
            out = orc.mxfp4_moe(x, w13, w13s, w2.reshape(E, K, N // 2), w2s.reshape(E, K, N // 32),
                                ids, wts)
            assert (out == 0).all(), (zb, e)


def test_moe_single_expert_is_gemv_act_gemv(orc):
    r = np.random.default_rng(1)
    hidden, inter, tokens = 64, 96, 3
    x = synth.bf16_normal(r, (tokens, hidden))
    w13, w13s = synth.mxfp4_matrix(r, 2 * inter, hidden)
    w2, w2s = synth.mxfp4_matrix(r, hidden, inter)
    ids = np.zeros((tokens, 1), dtype=np.int32)
    wts = np.ones((tokens, 1), dtype=np.float32)
    got = orc.mxfp4_moe_f64(x, w13[None], w13s[None], w2[None], w2s[None], ids, wts)
    h = orc.mxfp4_gemv_f64(w13, w13s, x)                      # [tokens, 2*inter]
    gate, up = h[:, :inter], h[:, inter:]
    a = gate * expit(gate) * up                               # silu via scipy's logistic
    y = a @ dense_mxfp4(orc, w2, w2s).T
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-12)


def test_moe_brute_force_tiny(orc):
    r = np.random.default_rng(5)
    E, hidden, inter, tokens, topk = 3, 32, 64, 5, 2
    x = synth.bf16_normal(r, (tokens, hidden))
    w13, w13s = synth.mxfp4_matrix(r, E * 2 * inter, hidden)
    w2, w2s = synth.mxfp4_matrix(r, E * hidden, inter)
    ids, wts = synth.router(r, tokens, E, topk)
    w13, w13s = w13.reshape(E, 2 * inter, -1), w13s.reshape(E, 2 * inter, -1)
    w2, w2s = w2.reshape(E, hidden, -1), w2s.reshape(E, hidden, -1)
    got = orc.mxfp4_moe_f64(x, w13, w13s, w2, w2s, ids, wts)
    xv = orc.f64_from_bf16(x)
    want = np.zeros((tokens, hidden))
    for t in range(tokens):
        for j in range(topk):
            e = ids[t, j]
            h = dense_mxfp4(orc, w13[e], w13s[e]) @ xv[t]
            a = h[:inter] * expit(h[:inter]) * h[inter:]
            want[t] += np.float64(wts[t, j]) * (dense_mxfp4(orc, w2[e], w2s[e]) @ a)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # permuting the slots of a token permutes nothing in the result
    got2 = orc.mxfp4_moe_f64(x, w13, w13s, w2, w2s, ids[:, ::-1], wts[:, ::-1])
    np.testing.assert_allclose(got2, got, rtol=1e-13, atol=1e-13)


def test_moe_rejects_bad_expert_ids(orc):
    r = np.random.default_rng(6)
    x = synth.bf16_normal(r, (1, 32))
    w13, w13s = synth.mxfp4_matrix(r, 64, 32)
    w2, w2s = synth.mxfp4_matrix(r, 32, 32)
    with pytest.raises(ValueError):
        orc.mxfp4_moe(x, w13[None], w13s[None], w2[None], w2s[None],
                      np.array([[1]], dtype=np.int32), np.ones((1, 1), np.float32))


# ------------------------------------------------------- small-batch ternary --

@pytest.mark.parametrize("batch,n,k", [(1, 9, 64), (3, 17, 256), (16, 40, 512)])
def test_ternary_gemm_matches_dense_product(orc, batch, n, k):
    """Each output row is the scaled ternary product of its activation row: a
    dense fp64 matmul of the decode (from the page's packing rule, applied in
    the encode direction here) against all rows at once."""
    r = np.random.default_rng(batch * 100 + n)
    t = r.integers(-1, 2, size=(n, k))
    s = r.uniform(0.01, 0.1, n).astype(np.float32)
    x = r.standard_normal((batch, k)).astype(np.float32)
    y, y64 = orc.ternary_gemm(pack_ternary(t), s, x, want_f64=True)
    want = (x.astype(np.float64) @ t.T.astype(np.float64)) * s.astype(np.float64)[None, :]
    bound = 1e-13 * (np.abs(x).astype(np.float64) @ np.abs(t).T) * s[None, :]
    assert (np.abs(y64 - want) <= bound).all()
    assert np.array_equal(y, y64.astype(np.float32))


def test_ternary_gemm_rows_are_independent(orc):
    """Permuting the activation rows permutes the output rows, and a zero row gives zeros."""
    case = synth.ternary_batch_case(5, 6, 64, 1024)
    perm = np.array([3, 0, 5, 1, 4, 2])
    x = case["x"].copy()
    x[4] = 0
    y = orc.ternary_gemm(case["packed"], case["row_scale"], x)
    yp = orc.ternary_gemm(case["packed"], case["row_scale"], x[perm])
    assert np.array_equal(yp, y[perm]) and (y[4] == 0).all()


def test_results_do_not_depend_on_the_thread_count(orc):
    """The CPU baseline times the oracle on one thread and on all of them: OpenMP splits
    rows only, never a sum, so both give the same bits."""
    case = synth.mxfp4_gemv_case(77, 96, 512, 2)
    tc = synth.ternary_case(78, 64, 512)
    xt = np.random.default_rng(79).standard_normal((3, 512)).astype(np.float32)
    n0 = orc.threads()
    try:
        orc.set_threads(1)
        one = (orc.mxfp4_gemv_f64(case["packed"], case["scales"], case["x"]),
               orc.ternary_gemm(tc["packed"], tc["row_scale"], xt, want_f64=True)[1])
        assert orc.threads() == 1
        orc.set_threads(max(2, n0))
        many = (orc.mxfp4_gemv_f64(case["packed"], case["scales"], case["x"]),
                orc.ternary_gemm(tc["packed"], tc["row_scale"], xt, want_f64=True)[1])
    finally:
        orc.set_threads(n0)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)
