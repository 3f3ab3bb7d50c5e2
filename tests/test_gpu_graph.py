"""Every entry point captured into one HIP graph and replayed (both N:M
kernels: the compiled 2:4 path and the generic one).

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
    tb = synth.ternary_batch_case(6, batch=3, n=320, k=1024)
    wl = synth.ternary_wl_case(7, n=256, k=1024)
    gg = synth.mxfp4_gemv_case(8, 200, 512, 130)              # prefill GEMM: 130 rows of x
    qx = synth.bf16_normal(r, (64, 256))
    # N:M weights: bf16 values and random position words (M a power of two: every field is valid)
    nmv = synth.bf16_normal(r, (300, 512), 0.02)               # 2:4, k = 1024
    nmm = r.integers(0, 2**32, size=(300, 32), dtype=np.uint64).astype(np.uint32)
    nmx = synth.bf16_normal(r, (2, 1024))
    ngv = synth.bf16_normal(r, (70, 3 * 48), 0.02)            # 3:16 (generic kernel), k = 768, batch 5
    ngm = r.integers(0, 2**32, size=(70, 18), dtype=np.uint64).astype(np.uint32)
    ngx = synth.bf16_normal(r, (5, 768))

    ins = {
        "gp": u8(gm["packed"]), "gs": u8(gm["scales"]), "gx": bf16(gm["x"]),
        "g4p": u8(g4["packed"]), "g4s": u8(g4["scales"]), "g4x": bf16(g4["x"]),
        "tp": words(tc["packed"]), "ts": f32(tc["row_scale"]), "tx": f32(tc["x"]),
        "table": u8(table), "bsc": u8(bsc), "gsc": f32(np.array([0.01], np.float32)), "ids": i64(ids),
        "mx": bf16(mc["x"]), "w13": u8(mc["w13"]), "w13s": u8(mc["w13_scale"]), "w2": u8(mc["w2"]),
        "w2s": u8(mc["w2_scale"]), "mid": i32(mc["topk_ids"]), "mw": f32(mc["topk_weights"]),
        "tbp": words(tb["packed"]), "tbs": f32(tb["row_scale"]), "tbx": f32(tb["x"]),
        "wlp": words(wl["packed"]), "wls": f32(wl["scale"]), "wlr": f32(wl["x_re"]), "wli": f32(wl["x_im"]),
        "ggp": u8(gg["packed"]), "ggs": u8(gg["scales"]), "ggx": bf16(gg["x"]),
        "qx": bf16(qx), "qg": f32(np.array([0.02], np.float32)),
        "nmv": bf16(nmv), "nmm": words(nmm), "nmx": bf16(nmx),
        "ngv": bf16(ngv), "ngm": words(ngm), "ngx": bf16(ngx),
    }
    outs = {
        "dec": torch.empty((1000, 4096), dtype=torch.bfloat16, device=dev),
        "y1": torch.empty((1, 1000), dtype=torch.bfloat16, device=dev),
        "y4": torch.empty((4, 300), dtype=torch.float32, device=dev),
        "yt": torch.empty((512,), dtype=torch.float32, device=dev),
        "emb": torch.empty((77, 2048), dtype=torch.bfloat16, device=dev),
        "moe": torch.empty((24, 256), dtype=torch.bfloat16, device=dev),
        "ytb": torch.empty((3, 320), dtype=torch.float32, device=dev),
        "wlr": torch.empty((256,), dtype=torch.float32, device=dev),
        "wli": torch.empty((256,), dtype=torch.float32, device=dev),
        "ygg": torch.empty((130, 200), dtype=torch.bfloat16, device=dev),
        "mxc": torch.empty((64, 128), dtype=torch.uint8, device=dev),
        "mxs": torch.empty((64, 8), dtype=torch.uint8, device=dev),
        "nvc": torch.empty((64, 128), dtype=torch.uint8, device=dev),
        "nvs": torch.empty((64, 16), dtype=torch.uint8, device=dev),
        "ynm": torch.empty((2, 300), dtype=torch.float32, device=dev),
        "yng": torch.empty((5, 70), dtype=torch.bfloat16, device=dev),
    }
    ws = torch.empty(gpu.mxfp4_moe_workspace_size(24, 256, 320, 8, 2), dtype=torch.uint8, device=dev)
    tws = torch.empty(gpu.ternary_gemm_workspace_size(ins["tbx"].shape[0], ins["tbp"].shape[0], ins["tbx"].shape[1]),
                      dtype=torch.uint8, device=dev)   # the digit pre-pass's buffer

    def run_all():
        gpu.dequant_decode(ins["gp"], ins["gs"], out=outs["dec"])
        gpu.dequant_gemv(ins["gp"], ins["gs"], ins["gx"], out_dtype=torch.bfloat16, out=outs["y1"])
        gpu.dequant_gemv(ins["g4p"], ins["g4s"], ins["g4x"], out=outs["y4"])
        gpu.ternary_gemv(ins["tp"], ins["ts"], ins["tx"], out=outs["yt"])
        gpu.nvfp4_embedding_gather(ins["table"], ins["bsc"], ins["gsc"], ins["ids"], out=outs["emb"])
        gpu.mxfp4_moe_gemm(ins["mx"], ins["w13"], ins["w13s"], ins["w2"], ins["w2s"], ins["mid"], ins["mw"],
                           out=outs["moe"], workspace=ws)
        gpu.ternary_gemm(ins["tbp"], ins["tbs"], ins["tbx"], out=outs["ytb"], workspace=tws)
        gpu.ternary_wl_gemv(ins["wlp"], ins["wls"], ins["wlr"], ins["wli"], out=(outs["wlr"], outs["wli"]))
        gpu.dequant_gemm(ins["ggp"], ins["ggs"], ins["ggx"], out=outs["ygg"])
        gpu.mxfp4_quantize(ins["qx"], out=(outs["mxc"], outs["mxs"]))
        gpu.nvfp4_quantize(ins["qx"], ins["qg"], out=(outs["nvc"], outs["nvs"]))
        gpu.nm_spmm(ins["nmv"], ins["nmm"], ins["nmx"], 2, 4, out=outs["ynm"])
        gpu.nm_spmm(ins["ngv"], ins["ngm"], ins["ngx"], 3, 16, out=outs["yng"])

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
            v.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
