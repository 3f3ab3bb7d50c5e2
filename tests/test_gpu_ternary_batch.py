"""GPU parity of ternary_gemm (small-batch ternary GEMM) against the oracle.

Tolerance, derived from the arithmetic of the fast kernel: it sums ternary
weights times a fixed-point rendering of each activation row exactly in int32
(per row and 256-column slice, x 2^S = H + L 2^-30 with |x 2^S| < 2^30: every
element of at least 2^-36 M_b is exact and any other is off by at most
2^-60 M_b, M_b the largest |x| of row b), then rounds at most k/256 + 24
times in fp32 (slice sums, digit columns, waves, the row scale), each at most
2^-23 of the row's magnitude. Element by element,
    |y - y_oracle| <= (k/256 + 24) 2^-23 s sum_c |t_c x_b,c| + 2^-60 M_b s sum_c |t_c| + 2^-23 |y_oracle|,
and the relative L2 error over the output stays below 2e-6. Inputs that take
the per-row ternary GEMV instead (K not a multiple of 64, unaligned weights)
are held to that kernel's bar, rel-L2 <= 1e-3 (plain fp32 adds of x).

Covers the 4096 x 4096 matrix at every batch 1..16, ragged row tiles and
slices, several slices per wave, workgroups that loop over tiles, rows of
very different magnitude (one exponent per row and slice), all-zero rows,
every field position with exact results, the fallback path, empty extents,
determinism, the digit workspace (uninitialised, reused, too small), and more
than 2 GiB of weights (sampled rows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import f32, host_f32, rel_l2, say, words

pytestmark = pytest.mark.gpu


def row_sums(packed, x):
    """Per (batch row, output row): sum_c |t_c| |x_b,c| and sum_c |t_c|, from the page's packing rule."""
    n, w = packed.shape
    ax = np.abs(x.astype(np.float64))
    mag = np.zeros((x.shape[0], n))
    cnt = np.zeros(n)
    for j in range(16):
        f = (packed >> np.uint32(2 * j)) & np.uint32(3)
        nz = ((f == 1) | (f == 2)).astype(np.float64)
        mag += ax[:, j::16] @ nz.T
        cnt += nz.sum(axis=1)
    return mag, cnt


def run(g, case, packed_dev=None):
    batch = case["x"].shape[0]
    n = case["packed"].shape[0]
    out = torch.full((batch, n), float("nan"), device="cuda:0")
    p = words(case["packed"]) if packed_dev is None else packed_dev
    g.ternary_gemm(p, f32(case["row_scale"]), f32(case["x"]), out=out)
    return host_f32(out)


def check(g, orc, case, packed_dev=None, fast=True):
    batch, k = case["x"].shape
    n = case["packed"].shape[0]
    say(f"ternary_gemm: batch={batch} n={n} k={k}")
    got = run(g, case, packed_dev)
    _, want = orc.ternary_gemm(case["packed"], case["row_scale"], case["x"], want_f64=True)
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    if fast:
        mag, cnt = row_sums(case["packed"], case["x"])
        s = np.abs(case["row_scale"].astype(np.float64))[None, :]
        M = np.abs(case["x"]).max(axis=1).astype(np.float64)[:, None]
        bound = (k / 256 + 24) * 2.0 ** -23 * s * mag + 2.0 ** -60 * M * s * cnt[None, :] + 2.0 ** -23 * np.abs(want)
        assert (np.abs(got - want) <= bound).all()
        assert err <= 2e-6, err
    else:
        assert err <= 1e-3, err
    return err


@pytest.mark.parametrize("batch", range(1, 17))
def test_workload_4096_every_batch(gpu, orc, batch):
    check(gpu, orc, synth.ternary_batch_case(synth.SEED_BASE + 6 + batch, batch, 4096, 4096))


@pytest.mark.parametrize("batch,n,k", [
    (3, 5, 64),           # one wave, one chunk
    (5, 33, 640),         # three waves, ragged last slice
    (8, 70, 2048),        # eight waves
    (2, 129, 4096 + 192), # sixteen waves, two slices for the first waves
    (16, 40, 8192),       # two slices per wave, four row groups
    (7, 17, 8192 + 64),   # three slices for wave 0, one chunk in the last
    (4, 40000, 1024),     # more tiles than resident workgroups
    (11, 9000, 4096 + 64),
    (6, 50, 64),          # one slice from batch 5 on: the second half of the slices is empty and adds +0
    (9, 31, 256),         # one full slice, odd batch
])
def test_fast_kernel_shapes(gpu, orc, batch, n, k):
    check(gpu, orc, synth.ternary_batch_case(batch * 1000 + n + k, batch, n, k))


def test_rows_of_different_magnitude_and_zero_rows(gpu, orc):
    case = synth.ternary_batch_case(31, 12, 300, 4096)
    x = case["x"].astype(np.float64)
    for b in range(12):
        x[b] *= 2.0 ** (3 * b - 18)
    x[5] = 0.0
    case["x"] = x.astype(np.float32)
    check(gpu, orc, case)
    got = run(gpu, case)
    assert (got[5] == 0).all()


@pytest.mark.parametrize("batch,n,k", [(3, 9, 16 * 37), (2, 50, 4096 + 16)])
def test_fallback_shapes(gpu, orc, batch, n, k):
    check(gpu, orc, synth.ternary_batch_case(batch * 77 + k, batch, n, k), fast=False)


def test_unaligned_weights_take_the_fallback(gpu, orc):
    case = synth.ternary_batch_case(41, 3, 24, 256)
    flat = np.zeros(case["packed"].size + 1, np.uint32)
    flat[1:] = case["packed"].reshape(-1)
    check(gpu, orc, case, packed_dev=words(flat)[1:].view(24, 16), fast=False)


def test_every_field_position_is_exact(gpu):
    """+1 / -1 at column i in rows 2i / 2i+1, scale 1: activation row b gives
    +/- x[b, i] exactly."""
    say("ternary_gemm: field positions")
    k, batch = 128, 5
    x = (np.arange(batch * k, dtype=np.float32).reshape(batch, k) - 300) * np.float32(0.125)
    P = np.zeros((2 * k, k // 16), dtype=np.uint32)
    for i in range(k):
        w, j = divmod(i, 16)
        P[2 * i, w] = np.uint32(1 << (2 * j + 1))
        P[2 * i + 1, w] = np.uint32(1 << (2 * j))
    got = run(gpu, {"packed": P, "row_scale": np.ones(2 * k, np.float32), "x": x})
    assert np.array_equal(got[:, 0::2], x) and np.array_equal(got[:, 1::2], -x)


def test_empty_and_deterministic(gpu):
    say("ternary_gemm: empty, determinism")
    y = torch.full((2, 4), 3.0, device="cuda:0")
    gpu.ternary_gemm(words(np.zeros((4, 0), np.uint32)), f32(np.ones(4, np.float32)),
                     torch.zeros((2, 0), device="cuda:0"), out=y)
    assert (host_f32(y) == 0).all()
    e = gpu.ternary_gemm(words(np.zeros((0, 4), np.uint32)), torch.zeros(0, device="cuda:0"),
                         torch.zeros((3, 64), device="cuda:0"))
    assert e.shape == (3, 0)
    case = synth.ternary_batch_case(8, 6, 512, 4096)
    assert np.array_equal(run(gpu, case), run(gpu, case))


def test_workspace_needs_no_initialisation_and_is_reusable(gpu):
    """From batch 5 on the fixed-point digits are prepared in the caller's workspace by a launch
    of their own. One buffer sized for batch 16 and filled with 0xFF serves a batch-16 call and
    then a batch-9 call (odd: the last group's second row lies past the batch) over a ragged last
    slice; each result is bit-identical to a call with a freshly allocated workspace. A workspace
    one byte short is refused."""
    say("ternary_gemm: workspace reuse")
    n, k = 300, 4096 + 64 * 3
    ws = torch.full((gpu.ternary_gemm_workspace_size(16, n, k),), 0xFF, dtype=torch.uint8, device="cuda:0")
    for batch in (16, 9):
        case = synth.ternary_batch_case(40 + batch, batch, n, k)
        fresh = run(gpu, case)
        out = torch.full((batch, n), float("nan"), device="cuda:0")
        gpu.ternary_gemm(words(case["packed"]), f32(case["row_scale"]), f32(case["x"]), out=out, workspace=ws)
        assert np.array_equal(host_f32(out), fresh), batch
    short = ws[:gpu.ternary_gemm_workspace_size(9, n, k) - 1]
    with pytest.raises(gpu.E2M1Error):
        gpu.ternary_gemm(words(case["packed"]), f32(case["row_scale"]), f32(case["x"]), workspace=short)


@pytest.mark.slow
@pytest.mark.parametrize("batch", [1, 4, 16])
def test_more_than_2_gib_of_weights(gpu, orc, batch):
    """540000 x 16384: 2.21 GB of packed weights, so the word offsets of the rows past 524287
    are beyond the 32-bit byte range. The first and last 64 output rows are held to the fast
    kernel's element bound against the oracle run on just those rows."""
    n, k = 540_000, 16384
    r = np.random.default_rng(synth.SEED_BASE + 91 + batch)
    w = r.integers(0, 1 << 32, (n, k // 16), dtype=np.uint32)
    np.bitwise_xor(w, (w >> np.uint32(1)) & w & np.uint32(0x55555555), out=w)   # field 3 -> 2: all valid
    case = {"packed": w, "row_scale": r.uniform(0.01, 0.1, size=n).astype(np.float32),
            "x": synth.f32_normal(r, (batch, k))}
    say(f"ternary_gemm: batch={batch} n={n} k={k} ({w.nbytes} bytes of weights)")
    got = run(gpu, case)
    sel = np.r_[0:64, n - 64:n]
    sub = {"packed": w[sel], "row_scale": case["row_scale"][sel], "x": case["x"]}
    _, want = orc.ternary_gemm(sub["packed"], sub["row_scale"], sub["x"], want_f64=True)
    g = got[:, sel]
    mag, cnt = row_sums(sub["packed"], sub["x"])
    s = np.abs(sub["row_scale"].astype(np.float64))[None, :]
    M = np.abs(sub["x"]).max(axis=1).astype(np.float64)[:, None]
    bound = (k / 256 + 24) * 2.0 ** -23 * s * mag + 2.0 ** -60 * M * s * cnt[None, :] + 2.0 ** -23 * np.abs(want)
    assert np.isfinite(got).all()
    assert (np.abs(g - want) <= bound).all()
    assert rel_l2(g, want) <= 2e-6
