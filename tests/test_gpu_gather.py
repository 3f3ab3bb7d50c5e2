"""GPU parity of nvfp4_embedding_gather: bit-exact against the oracle.

Covers the 200000 x 4096 table with 8192 ids (every gathered element), every
E4M3 scale byte against every code, the 16-channel path (hidden % 32 != 0),
ids outside the vocabulary (zero rows + flag), ids of any shape, the
empty call, and a table of more than 2 GiB of codes (sampled ids). Outputs are poisoned before each launch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, f32, i64, say, u8

pytestmark = pytest.mark.gpu


def run_gather(g, table, bscale, gscale, ids, flag=None):
    hidden = 2 * table.shape[1]
    out = torch.full((*np.shape(ids), hidden), -1, dtype=torch.int16, device="cuda:0")
    g.nvfp4_embedding_gather(u8(table), u8(bscale), f32(np.array([gscale], np.float32)),
                             i64(np.asarray(ids)), out=out, err_flag=flag)
    return bits(out)


@pytest.mark.slow
def test_workload_200k_vocab(gpu, orc):
    say("gather: 200000 x 4096 table, 8192 ids")
    c = synth.nvfp4_case()
    got = run_gather(gpu, c["table"], c["block_scale"], c["global_scale"], c["ids"])
    want, bad = orc.nvfp4_gather(c["table"], c["block_scale"], c["global_scale"], c["ids"])
    assert bad == 0
    assert np.array_equal(got, want)


def test_every_scale_byte_and_code(gpu, orc):
    say("gather: all 256 scale bytes x 16 codes")
    # row b: scale byte b in every group; the row holds all 256 byte values = all code pairs
    table = np.tile(np.arange(256, dtype=np.uint8), (256, 1))        # hidden 512
    bscale = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 32, axis=1)
    ids = np.arange(256, dtype=np.int64)
    # 1e-39: products in the bf16 subnormal range; 1e37 and 3e38: products and eff overflow to
    # infinity (a zero code then gives NaN, written as 0x7FC0)
    for gs in (0.01, 1.0, 0.37, 1e-39, 1e37, 3e38):
        got = run_gather(gpu, table, bscale, gs, ids)
        want, _ = orc.nvfp4_gather(table, bscale, gs, ids)
        assert np.array_equal(got, want), gs


@pytest.mark.parametrize("vocab,hidden,ntok", [(50, 16, 7), (300, 48, 33), (1000, 2048 + 32, 129),
                                               (64, 4096, 1), (10, 272, 64)])
def test_shapes(gpu, orc, vocab, hidden, ntok):
    say(f"gather: vocab={vocab} hidden={hidden} ntok={ntok}")
    r = np.random.default_rng(vocab + hidden + ntok)
    table = synth.uniform_bytes(r, (vocab, hidden // 2))
    bscale = synth.e4m3_log2_uniform(r, (vocab, hidden // 16))
    ids = synth.token_ids(r, ntok, vocab)
    got = run_gather(gpu, table, bscale, 0.01, ids)
    want, _ = orc.nvfp4_gather(table, bscale, 0.01, ids)
    assert np.array_equal(got, want)


def test_out_of_range_ids(gpu, orc):
    say("gather: out-of-range ids")
    r = np.random.default_rng(5)
    table = synth.uniform_bytes(r, (20, 64))
    bscale = synth.e4m3_log2_uniform(r, (20, 8))
    ids = np.array([[3, -1], [20, 19], [0, 2**40]], dtype=np.int64)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    got = run_gather(gpu, table, bscale, 0.01, ids, flag)
    want, bad = orc.nvfp4_gather(table, bscale, 0.01, ids.reshape(-1))
    assert bad == 3 and int(flag.item()) == 1
    assert np.array_equal(got.reshape(-1, 128), want)
    ok = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    run_gather(gpu, table, bscale, 0.01, np.array([0, 19]), ok)
    assert int(ok.item()) == 0


def test_empty(gpu):
    say("gather: empty")
    out = gpu.nvfp4_embedding_gather(u8(np.zeros((4, 8), np.uint8)), u8(np.zeros((4, 1), np.uint8)),
                                     f32(np.array([1.0], np.float32)),
                                     torch.zeros((0,), dtype=torch.int64, device="cuda:0"))
    assert out.shape == (0, 16)


def test_empty_vocabulary(gpu):
    """vocab == 0 with tokens: the table is never read (NULL is allowed), every row is zeros and
    the error flag is set (regression: the kernel used to read row 0 of the empty table)."""
    say("gather: empty vocabulary, NULL table, 5 ids")
    ids = torch.tensor([0, 1, -1, 7, 2**33], dtype=torch.int64, device="cuda:0")
    out = torch.full((5, 64), -1, dtype=torch.int16, device="cuda:0")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    gs = torch.tensor([0.01], dtype=torch.float32, device="cuda:0")
    lib = gpu.load_library()
    st = lib.nvfp4_embedding_gather(None, None, gs.data_ptr(), ids.data_ptr(), out.data_ptr(), 0, 64, 5,
                                    flag.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    assert int(torch.count_nonzero(out).item()) == 0
    # through the binding, with an empty (0, hidden/2) table
    flag.zero_()
    got = gpu.nvfp4_embedding_gather(torch.zeros((0, 32), dtype=torch.uint8, device="cuda:0"),
                                     torch.zeros((0, 4), dtype=torch.uint8, device="cuda:0"), gs, ids,
                                     err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    assert int(torch.count_nonzero(got.view(torch.int16)).item()) == 0


@pytest.mark.slow
def test_table_past_2_gib(gpu, orc):
    """1100000 x 4096: 2.25 GB of codes, so the rows past id 1048575 start beyond the 32-bit
    byte range. 96 ids (the first rows, the rows around 2^20, the last rows, random ones) are
    compared with the oracle run on just those rows."""
    vocab, hidden = 1_100_000, 4096
    r = np.random.default_rng(synth.SEED_BASE + 81)
    table = r.integers(0, 256, (vocab, hidden // 2), dtype=np.uint8)
    bscale = r.integers(0x20, 0x59, (vocab, hidden // 16), dtype=np.uint8)   # E4M3 2^-3 .. 2^4
    fixed = np.array([0, 1, 1048575, 1048576, 1048577, vocab - 2, vocab - 1], np.int64)
    ids = np.concatenate([fixed, r.integers(1_000_000, vocab, 89)]).astype(np.int64)
    say(f"gather: vocab={vocab} hidden={hidden} ({table.size} bytes of codes), {ids.size} ids")
    got = run_gather(gpu, table, bscale, 0.01, ids)
    uniq, local = np.unique(ids, return_inverse=True)
    want, bad = orc.nvfp4_gather(table[uniq], bscale[uniq], 0.01, local.astype(np.int64))
    assert bad == 0
    assert np.array_equal(got, want)
