"""Seeded synthetic inputs for the low-bit dequantisation workloads.

Shared by the tests, the smoke check and the benchmark. This module holds none
of the method's arithmetic: it only draws random bytes, integers and normals
(NumPy ``default_rng``), casts floats to bf16 / float8 with torch's own CPU
casts, and packs randomly drawn 2-bit patterns into words. It does not decode
anything and does not know which bit pattern means what.

Workload shapes (value distributions as stated for each):
  * MXFP4 GEMV, batch 1, W 256 x 512 (codes uniform over the 16 patterns, i.e.
    uniform bytes; one E8M0 byte per 32 columns uniform in 120..134; x bf16 of
    N(0,1)). Also a decode sweep of every byte over E8M0 100..150 and the zero
    bytes over all 256 exponents.
  * Ternary GEMV, W 4096 x 4096, each 2-bit pattern 00/01/10 with probability
    1/3; per-row fp32 scale U[0.01, 0.1]; x fp32 N(0,1).
  * Small-batch ternary GEMM: the ternary GEMV matrix with x fp32
    [batch, k] ~N(0,1), batch 1..16 (4 and 8 measured).
  * N:M structured-sparse weights (2:4 and 4:8 measured): bf16 values
    N(0, 0.02) with exactly N kept at uniformly random positions per group of
    M columns, x bf16 N(0, 1).
  * Widely-linear complex ternary layer, four such 4096 x 4096 matrices
    (U_re, U_im, W_re, W_im), four per-row scales U[0.01, 0.1], x_re and x_im
    fp32 N(0,1).
  * NVFP4 gather, table 200000 x 4096 (uniform bytes), E4M3 block scale per 16
    columns = 2^u with u ~ U[-4, 4] cast to float8_e4m3fn, global scale
    fp32(0.01), 8192 token ids uniform over the vocabulary.
  * MXFP4 GEMV in Llama-8B MLP shapes: 14336 x 4096 and 4096 x 14336, batch
    1, 4 or 16.
  * MXFP4 MoE: 32 experts, hidden = intermediate = 2880, 256 tokens, router
    logits N(0,1) -> top-4 experts, softmax over the selected four.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_BASE = 1000


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ------------------------------------------------------------- primitives --

def bf16_normal(r: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 N(0, std^2) draws, via torch's RNE cast."""
    f = r.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        f = f * np.float32(std)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_normal(r: np.random.Generator, shape) -> np.ndarray:
    return r.standard_normal(size=shape, dtype=np.float32)


def uniform_bytes(r: np.random.Generator, shape) -> np.ndarray:
    return r.integers(0, 256, size=shape, dtype=np.uint8)


def byte_range(r: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as uint8."""
    return r.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def mxfp4_matrix(r: np.random.Generator, n: int, k: int, e_lo: int = 120, e_hi: int = 134):
    """(packed uint8 [n, k/2], E8M0 uint8 [n, k/32]): uniform bytes, scales in [e_lo, e_hi]."""
    assert k % 32 == 0
    return uniform_bytes(r, (n, k // 2)), byte_range(r, (n, k // 32), e_lo, e_hi)


def two_bit_words(r: np.random.Generator, n: int, k: int, patterns=(0, 1, 2)) -> np.ndarray:
    """uint32 [n, k/16]: field j of word i is drawn uniformly from `patterns`
    (2-bit values) and stored at bits 2j..2j+1."""
    assert k % 16 == 0
    fields = r.choice(np.asarray(patterns, dtype=np.uint32), size=(n, k // 16, 16))
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(fields << shifts, axis=2).astype(np.uint32)


def e4m3_log2_uniform(r: np.random.Generator, shape, lo: float = -4.0, hi: float = 4.0) -> np.ndarray:
    """float8_e4m3fn bytes of 2^u, u ~ U[lo, hi], cast with torch (RNE)."""
    u = r.uniform(lo, hi, size=shape)
    f = torch.from_numpy(np.exp2(u).astype(np.float32))
    return f.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def token_ids(r: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    return r.integers(0, vocab, size=n, dtype=np.int64)


def router(r: np.random.Generator, tokens: int, experts: int, topk: int):
    """Top-k routing from N(0,1) logits: (ids int32 [tokens, topk] in descending
    logit order, weights fp32 = softmax over the selected logits). Routing is an
    input of the MoE layer, prepared here with torch CPU ops."""
    logits = torch.from_numpy(r.standard_normal(size=(tokens, experts), dtype=np.float32))
    vals, idx = torch.topk(logits, topk, dim=1, largest=True, sorted=True)
    w = torch.softmax(vals, dim=1)
    return idx.to(torch.int32).numpy().copy(), w.numpy().astype(np.float32).copy()


# ------------------------------------------------------------ workloads ----

def mxfp4_gemv_case(seed: int, n: int, k: int, batch: int = 1, e_lo: int = 120, e_hi: int = 134):
    r = rng(seed)
    packed, scales = mxfp4_matrix(r, n, k, e_lo, e_hi)
    x = bf16_normal(r, (batch, k))
    return {"packed": packed, "scales": scales, "x": x}


def gemv_small(seed: int = SEED_BASE + 0):
    """MXFP4 GEMV, batch 1, W 256 x 512."""
    return mxfp4_gemv_case(seed, 256, 512, 1)


def decode_sweep_all_bytes(e_lo: int = 100, e_hi: int = 150):
    """Every byte value 0..255 in each row; row i uses E8M0 = e_lo + i for all
    its blocks. Returns (packed [rows, 256], scales [rows, 16])."""
    exps = np.arange(e_lo, e_hi + 1, dtype=np.uint8)
    packed = np.tile(np.arange(256, dtype=np.uint8), (exps.size, 1))
    scales = np.repeat(exps[:, None], 512 // 32, axis=1).astype(np.uint8)
    return packed, scales


def decode_sweep_zero_bytes():
    """The four bytes made only of zero codes, repeated, at every E8M0 value:
    row e uses scale e. Returns (packed [256, 64], scales [256, 4])."""
    zero_bytes = np.array([0x00, 0x08, 0x80, 0x88], dtype=np.uint8)
    packed = np.tile(np.tile(zero_bytes, 16), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 4, axis=1)
    return packed, scales


def ternary_case(seed: int = SEED_BASE + 1, n: int = 4096, k: int = 4096):
    r = rng(seed)
    packed = two_bit_words(r, n, k)
    scale = r.uniform(0.01, 0.1, size=n).astype(np.float32)
    x = f32_normal(r, (k,))
    return {"packed": packed, "row_scale": scale, "x": x}


def nm_case(seed: int = SEED_BASE + 7, n_keep: int = 2, m: int = 4, rows: int = 4096, k: int = 4096,
            batch: int = 1):
    """N:M sparse weights: bf16 N(0, 0.02) values, a 0/1 mask with exactly n_keep
    ones at uniformly random positions in every group of m columns, x bf16 [batch, k]."""
    r = rng(seed)
    dense = bf16_normal(r, (rows, k), 0.02)
    keys = r.random((rows, k // m, m))
    order = np.argsort(keys, axis=2)
    mask = np.zeros((rows, k // m, m), dtype=np.uint8)
    np.put_along_axis(mask, order[:, :, :n_keep], 1, axis=2)
    x = bf16_normal(r, (batch, k))
    return {"dense": dense, "mask": mask.reshape(rows, k), "x": x, "n": n_keep, "m": m}


def ternary_batch_case(seed: int = SEED_BASE + 6, batch: int = 4, n: int = 4096, k: int = 4096):
    """Ternary GEMM for a few activation rows (speculative decoding): the
    ternary GEMV matrix and scales, x fp32 [batch, k] ~N(0, 1)."""
    r = rng(seed)
    packed = two_bit_words(r, n, k)
    scale = r.uniform(0.01, 0.1, size=n).astype(np.float32)
    x = f32_normal(r, (batch, k))
    return {"packed": packed, "row_scale": scale, "x": x}


def ternary_wl_case(seed: int = SEED_BASE + 5, n: int = 4096, k: int = 4096):
    """Widely-linear complex ternary layer: four ternary matrices U_re, U_im,
    W_re, W_im [n, k] (weights -1/0/+1 at 1/3 each, packed 16 per word), four
    per-row scales uniform [0.01, 0.1], x_re and x_im ~N(0, 1)."""
    r = rng(seed)
    packed = np.stack([two_bit_words(r, n, k) for _ in range(4)])
    scale = r.uniform(0.01, 0.1, size=(4, n)).astype(np.float32)
    x_re = f32_normal(r, (k,))
    x_im = f32_normal(r, (k,))
    return {"packed": packed, "scale": scale, "x_re": x_re, "x_im": x_im}


def nvfp4_case(seed: int = SEED_BASE + 2, vocab: int = 200000, hidden: int = 4096,
               tokens: int = 8192, global_scale: float = 0.01):
    r = rng(seed)
    table = uniform_bytes(r, (vocab, hidden // 2))
    block_scale = e4m3_log2_uniform(r, (vocab, hidden // 16))
    ids = token_ids(r, tokens, vocab)
    return {"table": table, "block_scale": block_scale,
            "global_scale": np.float32(global_scale), "ids": ids}


LLAMA8B_MLP_SHAPES = ((14336, 4096), (4096, 14336))


def llama_mlp_case(seed: int = SEED_BASE + 3, batch: int = 1, shapes=LLAMA8B_MLP_SHAPES):
    """One MXFP4 weight per (N, K) shape with its own bf16 activations [batch, K]."""
    r = rng(seed)
    out = []
    for n, k in shapes:
        packed, scales = mxfp4_matrix(r, n, k)
        out.append({"packed": packed, "scales": scales, "x": bf16_normal(r, (batch, k))})
    return out


def moe_case(seed: int = SEED_BASE + 4, experts: int = 32, hidden: int = 2880, inter: int = 2880,
             tokens: int = 256, topk: int = 4):
    r = rng(seed)
    w13, w13s = mxfp4_matrix(r, experts * 2 * inter, hidden)
    w2, w2s = mxfp4_matrix(r, experts * hidden, inter)
    x = bf16_normal(r, (tokens, hidden))
    ids, wts = router(r, tokens, experts, topk)
    return {
        "x": x,
        "w13": w13.reshape(experts, 2 * inter, hidden // 2),
        "w13_scale": w13s.reshape(experts, 2 * inter, hidden // 32),
        "w2": w2.reshape(experts, hidden, inter // 2),
        "w2_scale": w2s.reshape(experts, hidden, inter // 32),
        "topk_ids": ids, "topk_weights": wts,
    }
