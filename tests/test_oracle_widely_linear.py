"""Pins of the oracle's widely-linear complex ternary layer, y = U x + W conj(x).

FairyFuse blog post, section "复杂值广泛线性层的融合核调度": the layer is a
widely-linear map of a complex vector and splits into eight coupled real
ternary GEMVs. The oracle computes the complex definition directly; these
checks tie it to things outside itself: a pure-Python complex loop on tiny
inputs, numpy's complex128 matmul of a decode written here from the page's
packing rule, the eight real sub-GEMVs of the page evaluated with the
separately pinned real ternary GEMV, one-hot weights worked out by hand for
every matrix and sign, and the linearity of U x and the anti-linearity of
W conj(x) under multiplication of x by i.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth

NAMES = ("U_re", "U_im", "W_re", "W_im")


def pack_ternary(t: np.ndarray) -> np.ndarray:
    """{-1, 0, +1} [n, k] -> uint32 [n, k/16] by the page's packing formula:
    word = sum_j [1(w_j = +1) 2^(2j+1) + 1(w_j = -1) 2^(2j)]."""
    n, k = t.shape
    out = np.zeros((n, k // 16), dtype=np.uint64)
    for j in range(16):
        col = t[:, j::16]
        out += (col == 1).astype(np.uint64) << np.uint64(2 * j + 1)
        out += (col == -1).astype(np.uint64) << np.uint64(2 * j)
    return out.astype(np.uint32)


def unpack_ternary(words: np.ndarray) -> np.ndarray:
    """Decode direction of the same rule: +1 where bit 2j+1 is set, -1 where bit 2j is."""
    n, w = words.shape
    t = np.zeros((n, 16 * w), dtype=np.int64)
    for j in range(16):
        plus = (words >> np.uint32(2 * j + 1)) & np.uint32(1)
        minus = (words >> np.uint32(2 * j)) & np.uint32(1)
        t[:, j::16] = plus.astype(np.int64) - minus.astype(np.int64)
    return t


def random_case(seed, n, k):
    r = np.random.default_rng(seed)
    t = r.integers(-1, 2, size=(4, n, k))
    scale = r.uniform(0.01, 0.1, size=(4, n)).astype(np.float32)
    x_re = r.standard_normal(k).astype(np.float32)
    x_im = r.standard_normal(k).astype(np.float32)
    return t, scale, x_re, x_im


def magnitude(t, scale, x_re, x_im):
    """Per-row sum of |term| over the layer: the scale of fp64 rounding errors."""
    ax = np.abs(x_re.astype(np.float64)) + np.abs(x_im.astype(np.float64))
    return sum(np.abs(scale[m].astype(np.float64))[:, None] * np.abs(t[m]) @ ax for m in range(4))


def test_brute_force_tiny(orc):
    t, scale, x_re, x_im = random_case(11, 3, 32)
    (yr, yi), (y64r, y64i) = orc.ternary_wl_gemv([pack_ternary(m) for m in t], scale, x_re, x_im,
                                                 want_f64=True)
    n, k = t.shape[1:]
    for r in range(n):
        acc = 0j
        for c in range(k):
            u = float(scale[0, r]) * int(t[0, r, c]) + 1j * float(scale[1, r]) * int(t[1, r, c])
            w = float(scale[2, r]) * int(t[2, r, c]) + 1j * float(scale[3, r]) * int(t[3, r, c])
            x = complex(float(x_re[c]), float(x_im[c]))
            acc += u * x + w * x.conjugate()
        assert y64r[r] == pytest.approx(acc.real, rel=0, abs=1e-13)
        assert y64i[r] == pytest.approx(acc.imag, rel=0, abs=1e-13)
        assert yr[r] == np.float32(y64r[r]) and yi[r] == np.float32(y64i[r])


@pytest.mark.parametrize("n,k", [(37, 640), (8, 4096)])
def test_matches_complex_matmul(orc, n, k):
    case = synth.ternary_wl_case(n * 7 + k, n, k)
    t = np.stack([unpack_ternary(m) for m in case["packed"]])
    s = case["scale"].astype(np.float64)
    U = s[0][:, None] * t[0] + 1j * (s[1][:, None] * t[1])
    W = s[2][:, None] * t[2] + 1j * (s[3][:, None] * t[3])
    x = case["x_re"].astype(np.float64) + 1j * case["x_im"].astype(np.float64)
    want = U @ x + W @ np.conj(x)
    _, (y64r, y64i) = orc.ternary_wl_gemv(case["packed"], case["scale"], case["x_re"], case["x_im"],
                                          want_f64=True)
    bound = 1e-13 * magnitude(t, case["scale"], case["x_re"], case["x_im"])
    assert (np.abs(y64r - want.real) <= bound).all()
    assert (np.abs(y64i - want.imag) <= bound).all()


def test_eight_real_sub_gemvs(orc):
    """The page's decomposition: with T(M) v the scaled real ternary GEMV,
    Re y = T(U_re) x_re - T(U_im) x_im + T(W_re) x_re + T(W_im) x_im and
    Im y = T(U_re) x_im + T(U_im) x_re - T(W_re) x_im + T(W_im) x_re."""
    case = synth.ternary_wl_case(3, 50, 1024)
    P, s, xr, xi = case["packed"], case["scale"], case["x_re"], case["x_im"]

    def T(m, v):
        return orc.ternary_gemv(P[m], s[m], v, want_f64=True)[1]

    want_re = T(0, xr) - T(1, xi) + T(2, xr) + T(3, xi)
    want_im = T(0, xi) + T(1, xr) - T(2, xi) + T(3, xr)
    _, (y64r, y64i) = orc.ternary_wl_gemv(P, s, xr, xi, want_f64=True)
    t = np.stack([unpack_ternary(m) for m in P])
    bound = 1e-13 * magnitude(t, s, xr, xi)
    assert (np.abs(y64r - want_re) <= bound).all()
    assert (np.abs(y64i - want_im) <= bound).all()


def test_real_input_and_real_matrices_reduce_to_the_real_gemv(orc):
    case = synth.ternary_wl_case(4, 33, 512)
    P = case["packed"].copy()
    P[1] = 0
    P[3] = 0
    zero = np.zeros_like(case["x_im"])
    (yr, yi), (y64r, y64i) = orc.ternary_wl_gemv(P, case["scale"], case["x_re"], zero, want_f64=True)
    a = orc.ternary_gemv(P[0], case["scale"][0], case["x_re"], want_f64=True)[1]
    b = orc.ternary_gemv(P[2], case["scale"][2], case["x_re"], want_f64=True)[1]
    assert np.allclose(y64r, a + b, rtol=0, atol=1e-13)
    assert (y64i == 0).all() and (yi == 0).all()


@pytest.mark.parametrize("m", range(4))
@pytest.mark.parametrize("sign", [1, -1])
def test_one_hot_weight_in_each_matrix(orc, m, sign):
    """A single weight sign at column c of matrix m, scale s, x_c = u + iv:
    U_re: s(u + iv); U_im: i s (u + iv) = s(-v + iu);
    W_re: s(u - iv);  W_im: i s (u - iv) = s(v + iu)."""
    k, c, s = 64, 37, 0.375
    u, v = 1.25, -2.5
    t = np.zeros((4, 1, k), dtype=np.int64)
    t[m, 0, c] = sign
    scale = np.full((4, 1), 0.0, dtype=np.float32)
    scale[m, 0] = s
    x_re = np.zeros(k, np.float32)
    x_im = np.zeros(k, np.float32)
    x_re[c], x_im[c] = u, v
    want = {0: (u, v), 1: (-v, u), 2: (u, -v), 3: (v, u)}[m]
    yr, yi = orc.ternary_wl_gemv([pack_ternary(q) for q in t], scale, x_re, x_im)
    assert yr[0] == sign * s * want[0] and yi[0] == sign * s * want[1], NAMES[m]


def test_u_is_linear_and_w_conj_is_antilinear(orc):
    """With W = 0, y(i x) = i y(x); with U = 0, y(i x) = -i y(x). i x has real
    part -x_im and imaginary part x_re."""
    case = synth.ternary_wl_case(6, 20, 256)
    P, s, xr, xi = case["packed"], case["scale"], case["x_re"], case["x_im"]
    for keep, rot in (((0, 1), 1), ((2, 3), -1)):
        Q = np.zeros_like(P)
        for m in keep:
            Q[m] = P[m]
        _, (ar, ai) = orc.ternary_wl_gemv(Q, s, xr, xi, want_f64=True)
        _, (br, bi) = orc.ternary_wl_gemv(Q, s, -xi, xr, want_f64=True)
        # i (ar + i ai) = -ai + i ar;  -i (ar + i ai) = ai - i ar
        assert np.allclose(br, -rot * ai, rtol=0, atol=1e-13)
        assert np.allclose(bi, rot * ar, rtol=0, atol=1e-13)
        assert np.abs(ar).max() > 0.1


def test_invalid_field_and_empty(orc):
    P = np.zeros((4, 2, 1), dtype=np.uint32)
    P[3, 1, 0] = 3 << 10
    with pytest.raises(ValueError):
        orc.ternary_wl_gemv(P, np.ones((4, 2), np.float32), np.ones(16, np.float32),
                            np.ones(16, np.float32))
    yr, yi = orc.ternary_wl_gemv(np.zeros((4, 3, 0), np.uint32), np.ones((4, 3), np.float32),
                                 np.zeros(0, np.float32), np.zeros(0, np.float32))
    assert (yr == 0).all() and (yi == 0).all()
