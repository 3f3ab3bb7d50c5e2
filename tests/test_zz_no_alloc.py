"""GPU check of mxfp4_moe_gemm_noalloc (the MoE layer on the library's fixed per-GPU
workspace, for callers that cannot allocate) against mxfp4_moe_gemm with a caller
workspace, through the C ABI: two calls in a row on the same GPU, the second with a
smaller problem (so it runs on whatever the first left in the shared array). Both
entry points launch the same deterministic kernels, so the outputs must be
bit-identical (stricter than the layer's rel-L2 1e-2 bar against the oracle, which
the first case also checks).
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16, bf16_values, bits, f32, i32, rel_l2, say, u8

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, c):
    x, w13, w13s = bf16(c["x"]), u8(c["w13"]), u8(c["w13_scale"])
    w2, w2s = u8(c["w2"]), u8(c["w2_scale"])
    ids, wts = i32(c["topk_ids"]), f32(c["topk_weights"])
    T, H = c["x"].shape
    E, two_i, _ = c["w13"].shape
    topk = c["topk_ids"].shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = lib.mxfp4_moe_workspace_size(T, H, two_i // 2, E, topk)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device="cuda:0")
    out_ws = torch.full((T, H), -1, dtype=torch.int16, device="cuda:0")
    out_na = torch.full((T, H), -2, dtype=torch.int16, device="cuda:0")
    args = [_ptr(x), _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s), _ptr(ids), _ptr(wts)]
    assert lib.mxfp4_moe_gemm(*args, _ptr(out_ws), _ptr(ws), need, T, H, two_i // 2, E, topk, stream) == 0
    assert lib.mxfp4_moe_gemm_noalloc(*args, _ptr(out_na), T, H, two_i // 2, E, topk, stream) == 0
    return bits(out_ws), bits(out_na)


def test_noalloc_matches_workspace_entry_point(gpu, orc):
    lib = gpu.load_library()
    say("moe noalloc: 32 experts, 2880 x 2880, 256 tokens, top-4")
    big = synth.moe_case()
    a, b = _both(lib, big)
    assert np.array_equal(a, b)
    want = bf16_values(orc.mxfp4_moe(big["x"], big["w13"], big["w13_scale"], big["w2"], big["w2_scale"],
                                     big["topk_ids"], big["topk_weights"]))
    assert rel_l2(bf16_values(b), want) <= 1e-2
    say("moe noalloc: then a smaller layer (4 experts, 160 x 224, 33 tokens, top-2)")
    small = synth.moe_case(77, 4, 160, 224, 33, 2)
    a, b = _both(lib, small)
    assert np.array_equal(a, b)
    say("moe noalloc: then a larger one again (8 experts, 2880 x 2880, 16 tokens, top-4)")
    a, b = _both(lib, synth.moe_case(78, 8, 2880, 2880, 16, 4))
    assert np.array_equal(a, b)
