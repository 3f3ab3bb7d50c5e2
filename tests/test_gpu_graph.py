"""Every entry point captured into one HIP graph and replayed.

Between replays the outputs are poisoned eagerly and the device synchronised;
each replay must reproduce the eager results bit for bit (all kernels are
deterministic). The library launches only kernels (no memset or copy nodes),
so a captured call is the same work as an eager one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16, f32, i32, i64, say, u8, words

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu):
    say("graph: capture all entry points")
    dev = "cuda:0"
    gm = synth.mxfp4_gemv_case(1, 1000, 4096, 1)
    g4 = synth.mxfp4_gemv_case(2, 300, 2048, 4)
    tc = synth.ternary_case(3, 512, 4096)
    r = np.random.default_rng(4)
    table = synth.uniform_bytes(r, (500, 1024))
    bsc = synth.e4m3_log2_uniform(r, (500, 128))
    ids = synth.token_ids(r, 77, 500)
    mc = synth.moe_case(5, 8, 256, 320, 24, 2)

    ins = {
        "gp": u8(gm["packed"]), "gs": u8(gm["scales"]), "gx": bf16(gm["x"]),
        "g4p": u8(g4["packed"]), "g4s": u8(g4["scales"]), "g4x": bf16(g4["x"]),
        "tp": words(tc["packed"]), "ts": f32(tc["row_scale"]), "tx": f32(tc["x"]),
        "table": u8(table), "bsc": u8(bsc), "gsc": f32(np.array([0.01], np.float32)), "ids": i64(ids),
        "mx": bf16(mc["x"]), "w13": u8(mc["w13"]), "w13s": u8(mc["w13_scale"]), "w2": u8(mc["w2"]),
        "w2s": u8(mc["w2_scale"]), "mid": i32(mc["topk_ids"]), "mw": f32(mc["topk_weights"]),
    }
    outs = {
        "dec": torch.empty((1000, 4096), dtype=torch.bfloat16, device=dev),
        "y1": torch.empty((1, 1000), dtype=torch.bfloat16, device=dev),
        "y4": torch.empty((4, 300), dtype=torch.float32, device=dev),
        "yt": torch.empty((512,), dtype=torch.float32, device=dev),
        "emb": torch.empty((77, 2048), dtype=torch.bfloat16, device=dev),
        "moe": torch.empty((24, 256), dtype=torch.bfloat16, device=dev),
    }
    ws = torch.empty(gpu.mxfp4_moe_workspace_size(24, 256, 320, 8, 2), dtype=torch.uint8, device=dev)

    def run_all():
        gpu.dequant_decode(ins["gp"], ins["gs"], out=outs["dec"])
        gpu.dequant_gemv(ins["gp"], ins["gs"], ins["gx"], out_dtype=torch.bfloat16, out=outs["y1"])
        gpu.dequant_gemv(ins["g4p"], ins["g4s"], ins["g4x"], out=outs["y4"])
        gpu.ternary_gemv(ins["tp"], ins["ts"], ins["tx"], out=outs["yt"])
        gpu.nvfp4_embedding_gather(ins["table"], ins["bsc"], ins["gsc"], ins["ids"], out=outs["emb"])
        gpu.mxfp4_moe_gemm(ins["mx"], ins["w13"], ins["w13s"], ins["w2"], ins["w2s"], ins["mid"], ins["mw"],
                           out=outs["moe"], workspace=ws)

    run_all()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        for v in outs.values():
            v.view(torch.int16 if v.element_size() == 2 else torch.int32).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
