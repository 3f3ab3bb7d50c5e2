"""GPU parity of ternary_wl_gemv (widely-linear complex ternary layer) against the oracle.

Tolerance, derived from the arithmetic of the fast kernel. It sums ternary
weights times a fixed-point rendering of x exactly in int32: per 256-column
slice and part, x 2^S = H + L 2^-30 with |x 2^S| < 2^30, so every element of
at least 2^-36 M is exact and any other is off by at most 2^-60 M (M = largest
|x| of that part over all of K). The integer sums then pass through at most k/256 + 32 fp32
roundings (slice sums, digit columns, waves, scales and the complex
combination), each at most 2^-23 (2u, to allow for an adder that truncates)
of the row's magnitude. Hence, element by element,
    |y - y_oracle| <= (k/256 + 32) 2^-23 mag + 2^-60 (M_re + M_im) cnt + 2^-23 |y_oracle|
with mag = sum_m s_m sum_c |t_mc| (|x_re,c| + |x_im,c|) and
cnt = sum_m s_m sum_c |t_mc|. The one-wave-per-row kernel (plain fp32 adds
of x) meets the same form with k roundings: its cases use (k + 32) in place
of (k/256 + 32). On top of that the relative L2 error must stay below 2e-6:
a correct kernel lands near 1e-7, while losing the fraction digits of x (x
kept to 30 bits below the slice maximum) or one fp32 piece would show at 1e-6
to 1e-5.

Covers the 4096 x 4096 layer (full output), one and several slices per wave,
workgroups that loop over tiles, ragged row tiles and slices, the
one-wave-per-row kernel (K not a multiple of 64, unaligned matrices), every
field position of every matrix with exact results, empty extents and
determinism.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import f32, host_f32, rel_l2, say, words

pytestmark = pytest.mark.gpu

REL_L2 = 2e-6


def magnitudes(case):
    """Per row: mag = sum_m s_m sum_c |t_mc| (|x_re,c| + |x_im,c|) and cnt = sum_m s_m sum_c |t_mc|."""
    ax = np.abs(case["x_re"].astype(np.float64)) + np.abs(case["x_im"].astype(np.float64))
    n = case["packed"].shape[1]
    mag = np.zeros(n, dtype=np.float64)
    cnt = np.zeros(n, dtype=np.float64)
    for m in range(4):
        P = case["packed"][m]
        row = np.zeros(n, dtype=np.float64)
        num = np.zeros(n, dtype=np.float64)
        for j in range(16):
            f = (P >> np.uint32(2 * j)) & np.uint32(3)
            nz = ((f == 1) | (f == 2)).astype(np.float64)
            row += nz @ ax[j::16]
            num += nz.sum(axis=1)
        sm = np.abs(case["scale"][m].astype(np.float64))
        mag += sm * row
        cnt += sm * num
    return mag, cnt


def bound(case, y64, generic=False):
    k = case["x_re"].shape[0]
    mag, cnt = magnitudes(case)
    big = float(np.abs(case["x_re"]).max(initial=0.0)) + float(np.abs(case["x_im"]).max(initial=0.0))
    steps = (k if generic else k / 256) + 32
    return steps * 2.0 ** -23 * mag + 2.0 ** -60 * big * cnt + 2.0 ** -23 * np.abs(y64)


def run(g, case, mats=None):
    P = case["packed"]
    n = P.shape[1]
    mats = [words(P[m]) for m in range(4)] if mats is None else mats
    out = (torch.full((n,), float("nan"), device="cuda:0"), torch.full((n,), float("nan"), device="cuda:0"))
    g.ternary_wl_gemv(mats, f32(case["scale"]), f32(case["x_re"]), f32(case["x_im"]), out=out)
    return host_f32(out[0]), host_f32(out[1])


def check(g, orc, case, mats=None, generic=False):
    n, w = case["packed"].shape[1:]
    say(f"ternary_wl: n={n} k={16 * w}")
    got_re, got_im = run(g, case, mats)
    (_, _), (w_re, w_im) = orc.ternary_wl_gemv(case["packed"], case["scale"], case["x_re"], case["x_im"],
                                               want_f64=True)
    assert np.isfinite(got_re).all() and np.isfinite(got_im).all()
    assert (np.abs(got_re - w_re) <= bound(case, w_re, generic)).all()
    assert (np.abs(got_im - w_im) <= bound(case, w_im, generic)).all()
    err = rel_l2(np.concatenate([got_re, got_im]), np.concatenate([w_re, w_im]))
    assert err <= REL_L2, err
    return err


def test_workload_4096(gpu, orc):
    check(gpu, orc, synth.ternary_wl_case())


@pytest.mark.parametrize("n,k", [
    (5, 64),            # one wave per workgroup, one chunk
    (33, 640),          # three waves, ragged last slice
    (70, 2048),         # eight waves
    (129, 4096 + 192),  # sixteen waves, two slices for the first waves
    (40, 8192),         # two slices per wave
    (17, 8192 + 64),    # three slices for wave 0, one chunk in the last
    (40000, 1024),      # more tiles than resident workgroups: tile loop
    (9000, 4096 + 64),  # tile loop with several slices per wave
])
def test_fast_kernel_shapes(gpu, orc, n, k):
    check(gpu, orc, synth.ternary_wl_case(n * 13 + k, n, k))


@pytest.mark.parametrize("n,k", [(9, 16 * 37), (3, 16), (50, 4096 + 16)])
def test_generic_kernel_shapes(gpu, orc, n, k):
    check(gpu, orc, synth.ternary_wl_case(n * 17 + k, n, k), generic=True)


def test_unaligned_matrix_takes_the_generic_kernel(gpu, orc):
    case = synth.ternary_wl_case(21, 24, 256)
    mats = []
    for m in range(4):
        flat = np.zeros(case["packed"][m].size + 1, np.uint32)
        flat[1:] = case["packed"][m].reshape(-1)
        mats.append(words(flat)[1:].view(24, 16))
    check(gpu, orc, case, mats=mats, generic=True)


@pytest.mark.parametrize("m", range(4))
def test_every_field_of_each_matrix_is_exact(gpu, m):
    """+1 / -1 at column i of matrix m in rows 2i / 2i+1, all scales 1: row
    results are the hand-worked entries of x times the unit weight."""
    say(f"ternary_wl: field positions, matrix {m}")
    k = 128
    x_re = np.arange(1, k + 1, dtype=np.float32) * np.float32(0.25)
    x_im = -np.arange(1, k + 1, dtype=np.float32) * np.float32(1.5) + np.float32(7.0)
    P = np.zeros((4, 2 * k, k // 16), dtype=np.uint32)
    for i in range(k):
        w, j = divmod(i, 16)
        P[m, 2 * i, w] = np.uint32(1 << (2 * j + 1))
        P[m, 2 * i + 1, w] = np.uint32(1 << (2 * j))
    case = {"packed": P, "scale": np.ones((4, 2 * k), np.float32), "x_re": x_re, "x_im": x_im}
    got_re, got_im = run(gpu, case)
    u, v = x_re.astype(np.float64), x_im.astype(np.float64)
    want = {0: (u, v), 1: (-v, u), 2: (u, -v), 3: (v, u)}[m]
    assert np.array_equal(got_re[0::2], want[0]) and np.array_equal(got_im[0::2], want[1])
    assert np.array_equal(got_re[1::2], -want[0]) and np.array_equal(got_im[1::2], -want[1])


def test_empty_and_deterministic(gpu):
    say("ternary_wl: empty, determinism")
    y = (torch.full((4,), 3.0, device="cuda:0"), torch.full((4,), 3.0, device="cuda:0"))
    z = torch.zeros((4, 0), dtype=torch.int32, device="cuda:0")
    gpu.ternary_wl_gemv([z, z, z, z], f32(np.ones((4, 4), np.float32)), torch.zeros(0, device="cuda:0"),
                        torch.zeros(0, device="cuda:0"), out=y)
    assert (host_f32(y[0]) == 0).all() and (host_f32(y[1]) == 0).all()
    e = torch.zeros((0, 4), dtype=torch.int32, device="cuda:0")
    r = gpu.ternary_wl_gemv([e, e, e, e], f32(np.ones((4, 0), np.float32)), torch.zeros(64, device="cuda:0"),
                            torch.zeros(64, device="cuda:0"))
    assert r[0].numel() == 0
    case = synth.ternary_wl_case(8, 512, 4096)
    a = run(gpu, case)
    b = run(gpu, case)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
