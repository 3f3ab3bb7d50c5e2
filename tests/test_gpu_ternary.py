"""GPU parity of ternary_gemv against the oracle (rel-L2 <= 1e-3; the fast path
sums exactly over a fixed-point x and must stay below 1e-5 at 4096 x 4096).

Covers the 4096 x 4096 workload (full output), one to sixteen waves per
workgroup and several slices per wave on the int8 matrix-core path, the
slower kernel (K not a multiple of 64, misaligned weights), misaligned x,
every bit position of a word, empty extents and determinism.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import f32, host_f32, rel_l2, say, words

pytestmark = pytest.mark.gpu

TOL = 1e-3


def ternary_case(g, orc, case, x_dev=None):
    n, w = case["packed"].shape
    say(f"ternary: n={n} k={16 * w}")
    out = torch.full((n,), float("nan"), device="cuda:0")
    x = f32(case["x"]) if x_dev is None else x_dev
    g.ternary_gemv(words(case["packed"]), f32(case["row_scale"]), x, out=out)
    got = host_f32(out)
    want = orc.ternary_gemv(case["packed"], case["row_scale"], case["x"])
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    assert err <= TOL, err
    return err


def test_workload_4096(gpu, orc):
    err = ternary_case(gpu, orc, synth.ternary_case())
    assert err < 1e-5


@pytest.mark.parametrize("n,k", [(5, 64), (33, 640), (70, 2048), (129, 4096 + 64 * 3), (40, 8192),
                                 (9, 16 * 37), (17, 8192 + 64), (3, 16)])
def test_shapes(gpu, orc, n, k):
    ternary_case(gpu, orc, synth.ternary_case(n * 13 + k, n, k))


def test_misaligned_x(gpu, orc):
    case = synth.ternary_case(4, 16, 256)
    xbig = torch.zeros(257, device="cuda:0")
    xbig[1:] = f32(case["x"])
    ternary_case(gpu, orc, case, x_dev=xbig[1:])


def test_misaligned_weights_take_the_slow_kernel(gpu, orc):
    case = synth.ternary_case(14, 20, 512)
    n, w = case["packed"].shape
    say(f"ternary: misaligned weights n={n} k={16 * w}")
    flat = np.zeros(case["packed"].size + 1, np.uint32)
    flat[1:] = case["packed"].reshape(-1)
    out = torch.full((n,), float("nan"), device="cuda:0")
    gpu.ternary_gemv(words(flat)[1:].view(n, w), f32(case["row_scale"]), f32(case["x"]), out=out)
    want = orc.ternary_gemv(case["packed"], case["row_scale"], case["x"])
    assert rel_l2(host_f32(out), want) <= TOL


def test_every_bit_position(gpu):
    say("ternary: bit positions")
    k = 64
    x = np.arange(1, k + 1, dtype=np.float32)
    packed = np.zeros((2 * k, k // 16), dtype=np.uint32)
    for i in range(k):
        w, j = divmod(i, 16)
        packed[2 * i, w] = np.uint32(1 << (2 * j + 1))      # +1 at column i
        packed[2 * i + 1, w] = np.uint32(1 << (2 * j))      # -1 at column i
    y = host_f32(gpu.ternary_gemv(words(packed), f32(np.ones(2 * k, np.float32)), f32(x)))
    assert np.array_equal(y[0::2], x) and np.array_equal(y[1::2], -x)


def test_empty_and_deterministic(gpu):
    say("ternary: empty, determinism")
    y = torch.full((4,), 3.0, device="cuda:0")
    gpu.ternary_gemv(words(np.zeros((4, 0), np.uint32)), f32(np.ones(4, np.float32)),
                     torch.zeros(0, device="cuda:0"), out=y)
    assert (host_f32(y) == 0).all()
    case = synth.ternary_case(8, 512, 4096)
    args = (words(case["packed"]), f32(case["row_scale"]), f32(case["x"]))
    assert np.array_equal(host_f32(gpu.ternary_gemv(*args)), host_f32(gpu.ternary_gemv(*args)))
