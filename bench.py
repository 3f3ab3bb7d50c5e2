#!/usr/bin/env python3
"""Benchmark of the low-bit dequantisation hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line. The default workload is the headline: MXFP4 dequant-GEMV
at batch 1 on the Llama-8B MLP shapes (W 14336 x 4096 and W 4096 x 14336, one
launch each per step), bf16 output. Other workloads (for the per-kernel
roofline tables): mlp_b2, mlp_b4, mlp_b8, mlp_b16, ternary, ternary_b1 .. ternary_b16
(small-batch ternary GEMM), ternary_wl, gather, moe, decode, decode_8192 (the
same bytes as the gather), quantize,
prefill (MXFP4 GEMM, 2048 tokens), nm_2of4, nm_4of8, gemv_small. Platform
reference points (libe2m1probe.so): floor (empty launches), stream_31mb and
stream_31mb_store (a plain read of the headline launch's 31.2 MB, without and
with a 4-byte store per wave), stream_31mb_store1 (one 4-byte store in all),
stream_4mb_store (the 4096 x 4096 ternary matrix's 4 MiB, with a store per wave),
stream_128mb, stream_512mb, mfma_peak.

Timing: inputs are resident in HBM before the timed region. The launches of
one step per weight copy are captured into a HIP graph; W warmup steps are
replayed untimed, then at least K steps (whole graph replays) are timed with
HIP events on torch's current stream, bracketed by torch.cuda.synchronize().
Each kernel's average duration for the roofline comes from a graph of that
kernel alone, timed the same way. Weight copies are rotated so that the bytes
cycled per replay exceed the 256 MB Infinity Cache: every launch reads its
weights from HBM.

`cpu_baseline` is the CPU oracle (plain C, fp64, OpenMP over rows) timed on a
bounded sample of the same workload on this host's cores, then again on one
core (`single_core`) -- a reported baseline, not a target.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "effective weight GB/s and % HBM peak, batch-1 low-bit dequant-GEMV"
CSRC = os.path.join(ROOT, "gemm_e2m1_lut_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# Source files each launch label's device code is built from (plus the shared
# device helpers): a counter summary stays valid only while these are unchanged.
# The declarations in kernels.hpp and the host-side checks in api.hip compile to
# no device code; each kernel's launch logic lives in its own source file.
KERNEL_SOURCES = {
    "probe": ["../probe/platform_probe.hip"],
    "gemv": ["gemv.hip"],
    "moe": ["moe.hip", "moe_engine.hpp"],
    "ternary": ["ternary.hip", "ternary_batch.hip", "ternary_int8.hpp"],
    "ternarywl": ["ternary_wl.hip", "ternary_int8.hpp"],
    "ternarygemm": ["ternary_batch.hip", "ternary_int8.hpp"],
    "gather": ["gather.hip"],
    "decode": ["decode.hip"],
    "mxquant": ["quantize.hip"],
    "gemm": ["gemm.hip"],
    "nvquant": ["quantize.hip"],
    "nm": ["nm_sparse.hip"],
}
COMMON_SOURCES = ["device.hpp"]


def _code_only(text: str) -> str:
    """Source text without comments and blank space: edits to comments leave the
    kernels, and so the counters taken for them, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())


def build_fingerprint(flags: list[str] | None = None, root: str | None = None) -> str:
    """The compiler flags and offload target the library is built with: a flag change alters
    the machine code (and so the counters) as much as a source edit does. Paths inside the
    checkout are written relative to it, so a copy of the tree elsewhere has the same
    fingerprint."""
    from gemm_e2m1_lut_amd import build as hip_build
    flags = hip_build.HIPFLAGS if flags is None else flags
    root = hip_build.ROOT if root is None else root
    return " ".join(f.replace(root, "<repo>") for f in flags)


def kernel_source_hash(label: str, flags: str | None = None) -> str:
    family = label.split("_")[0]
    h = hashlib.sha256()
    h.update((build_fingerprint() if flags is None else flags).encode())
    common = [] if family == "probe" else COMMON_SOURCES
    for name in sorted(KERNEL_SOURCES.get(family, []) + common):
        path = os.path.join(CSRC, name)
        if os.path.exists(path):
            with open(path, encoding="utf-8") as fh:
                h.update((name + _code_only(fh.read())).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------- workloads ---

class Workload:
    """One step = every launch in `launches` once, on weight copy `i % copies`."""
    name = ""
    config: dict = {}
    dtype = "bf16"
    bound = "hbm"

    def launches(self):  # -> list of (label, fn(copy_index))
        raise NotImplementedError

    def alg_bytes(self, label: str) -> float:  # algorithmic bytes of one launch
        raise NotImplementedError

    def alg_flops(self, label: str) -> float:
        return 0.0

    weight_bytes_per_step = 0.0
    total_bytes_per_step = 0.0
    # a reference-point workload reports its own metric instead of the headline's
    metric: str | None = None

    def cpu_baseline(self, budget_s: float) -> dict | None:
        return None

    def headline(self, ms_per_step: float, per_launch: dict) -> tuple[float, str, bool]:
        """(value, unit, higher_is_better) of the JSON line for a reference-point workload."""
        raise NotImplementedError


def _gen(seed: int):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _mxfp4_dev(g, n: int, k: int, lo: int = 120, hi: int = 134):
    import torch
    packed = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    scales = torch.randint(lo, hi + 1, (n, k // 32), dtype=torch.uint8, device="cuda", generator=g)
    return packed, scales


class GemvMLP(Workload):
    SHAPES = ((14336, 4096), (4096, 14336))

    def __init__(self, batch: int, rotate_bytes: float):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib = lib
        self.batch = batch
        self.name = f"llama8b_mlp_mxfp4_gemv_b{batch}"
        g = _gen(4242 + batch)
        per_copy = sum(n * k // 2 + n * k // 32 for n, k in self.SHAPES)
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.weights = [[_mxfp4_dev(g, n, k) for n, k in self.SHAPES] for _ in range(self.copies)]
        self.x = [torch.randn((batch, k), generator=g, device="cuda").to(torch.bfloat16)
                  for _, k in self.SHAPES]
        self.y = [torch.empty((batch, n), dtype=torch.bfloat16, device="cuda") for n, _ in self.SHAPES]
        self.weight_bytes_per_step = float(per_copy)
        self.total_bytes_per_step = float(sum(self.alg_bytes(l) for l, _ in self.launches()))
        self.config = {"workload": self.name, "shapes_NxK": [list(s) for s in self.SHAPES],
                       "batch": batch, "weights": "MXFP4 (E2M1 codes + E8M0 per 32)",
                       "activations": "bf16", "out": "bf16", "accumulate": "fp32",
                       "weight_copies_rotated": self.copies,
                       "rotated_MB": round(self.copies * per_copy / 1e6, 1)}

    def launches(self):
        out = []
        for j, (n, k) in enumerate(self.SHAPES):
            def fn(i, j=j):
                p, s = self.weights[i % self.copies][j]
                self.lib.dequant_gemv(p, s, self.x[j], out_dtype=self.y[j].dtype, out=self.y[j])
            out.append((f"gemv_b{self.batch}_{n}x{k}", fn))
        return out

    def alg_bytes(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return n * k // 2 + n * k // 32 + self.batch * k * 2 + self.batch * n * 2

    def alg_flops(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return 2.0 * self.batch * n * k

    def cpu_baseline(self, budget_s):
        import oracle
        host = [(p.cpu().numpy(), s.cpu().numpy()) for p, s in self.weights[0]]
        xs = [x.view(__import__("torch").int16).cpu().numpy().view(np.uint16) for x in self.x]
        reps, t0 = 0, time.perf_counter()
        while True:
            for (p, s), x in zip(host, xs):
                oracle.mxfp4_gemv_f64(p, s, x)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 200:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full step (both MLP shapes, batch {self.batch}) repeated {reps} times, "
                          f"{el:.1f} s, fp64 scalar C with OpenMP over rows"}


class GemvMLPGrouped(GemvMLP):
    """The batch-1 MLP step with both products in one dequant_gemv_grouped call (one launch)."""
    LABEL = "gemv_b1_grouped_14336x4096+4096x14336"

    def __init__(self, rotate_bytes: float):
        super().__init__(1, rotate_bytes)
        self.name = "llama8b_mlp_mxfp4_gemv_b1_grouped"
        self.config["workload"] = self.name
        self.config["launch"] = "both products in one dequant_gemv_grouped call"

    def launches(self):
        def fn(i):
            mats = [(p, s, x[0]) for (p, s), x in zip(self.weights[i % self.copies], self.x)]
            self.lib.dequant_gemv_grouped(mats, out_dtype=self.y[0].dtype, outs=[y[0] for y in self.y])
        return [(self.LABEL, fn)]

    def alg_bytes(self, label):
        return sum(n * k // 2 + n * k // 32 + k * 2 + n * 2 for n, k in self.SHAPES)

    def alg_flops(self, label):
        return sum(2.0 * n * k for n, k in self.SHAPES)


class Ternary(Workload):
    def __init__(self, rotate_bytes: float, n: int = 4096, k: int = 4096):
        import torch
        import gemm_e2m1_lut_amd as lib
        import synth
        self.lib, self.n, self.k = lib, n, k
        self.name = f"ternary_gemv_{n}x{k}"
        per_copy = n * k // 4
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        r = synth.rng(synth.SEED_BASE + 1)
        base = synth.two_bit_words(r, n, k)
        self.host = {"packed": base, "row_scale": r.uniform(0.01, 0.1, n).astype(np.float32),
                     "x": synth.f32_normal(r, (k,))}
        dev0 = torch.from_numpy(base.view(np.int32)).cuda()
        # rotated copies: the same weights rolled by whole rows (distinct addresses, same statistics)
        self.packed = [torch.roll(dev0, shifts=7 * i, dims=0).contiguous() for i in range(self.copies)]
        self.scale = torch.from_numpy(self.host["row_scale"]).cuda()
        self.x = torch.from_numpy(self.host["x"]).cuda()
        self.y = torch.empty(n, device="cuda")
        self.weight_bytes_per_step = float(per_copy + 4 * n)
        self.total_bytes_per_step = float(self.alg_bytes("ternary"))
        self.dtype = "f32"
        self.config = {"workload": self.name, "weights": "2-bit ternary, 16 per uint32",
                       "activations": "fp32", "out": "fp32", "weight_copies_rotated": self.copies}

    def launches(self):
        def fn(i):
            self.lib.ternary_gemv(self.packed[i % self.copies], self.scale, self.x, out=self.y)
        return [("ternary", fn)]

    def alg_bytes(self, label):
        return self.n * self.k // 4 + 4 * self.n + 4 * self.k + 4 * self.n

    def cpu_baseline(self, budget_s):
        import oracle
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.ternary_gemv(self.host["packed"], self.host["row_scale"], self.host["x"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 2000:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full 4096 x 4096 GEMV repeated {reps} times, {el:.1f} s"}


class TernaryBatch(Workload):
    """Small-batch ternary GEMM: the 4096 x 4096 ternary matrix against
    `batch` activation rows (speculative decoding)."""

    def __init__(self, batch: int, rotate_bytes: float, n: int = 4096, k: int = 4096):
        import torch
        import gemm_e2m1_lut_amd as lib
        import synth
        self.lib, self.batch, self.n, self.k = lib, batch, n, k
        self.name = f"ternary_gemm_b{batch}_{n}x{k}"
        per_copy = n * k // 4
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.host = synth.ternary_batch_case(batch=batch, n=n, k=k)
        dev0 = torch.from_numpy(self.host["packed"].view(np.int32)).cuda()
        # rotated copies: the same weights rolled by whole rows (distinct addresses, same statistics)
        self.packed = [torch.roll(dev0, shifts=7 * i, dims=0).contiguous() for i in range(self.copies)]
        self.scale = torch.from_numpy(self.host["row_scale"]).cuda()
        self.x = torch.from_numpy(self.host["x"]).cuda()
        self.y = torch.empty(batch, n, device="cuda")
        need = lib.ternary_gemm_workspace_size(batch, n, k)   # the digit pre-pass's buffer, made once
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need > 0 else None
        self.weight_bytes_per_step = float(per_copy + 4 * n)
        self.label = f"ternarygemm_b{batch}"
        self.total_bytes_per_step = float(self.alg_bytes(self.label))
        self.dtype = "f32"
        self.config = {"workload": self.name, "weights": "2-bit ternary, 16 per uint32", "batch": batch,
                       "activations": "fp32", "out": "fp32", "weight_copies_rotated": self.copies}

    def launches(self):
        def fn(i):
            self.lib.ternary_gemm(self.packed[i % self.copies], self.scale, self.x, out=self.y, workspace=self.ws)
        return [(self.label, fn)]

    def alg_bytes(self, label):
        return self.n * self.k // 4 + 4 * self.n + 4 * self.batch * (self.k + self.n)

    def cpu_baseline(self, budget_s):
        import oracle
        h = self.host
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.ternary_gemm(h["packed"], h["row_scale"], h["x"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 2000:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full {self.n} x {self.k} GEMM at batch {self.batch} repeated {reps} times, "
                          f"{el:.1f} s"}


class TernaryWL(Workload):
    """Widely-linear complex ternary layer y = U x + W conj(x): four ternary
    matrices (U_re, U_im, W_re, W_im) of n x k, four per-row scales."""

    def __init__(self, rotate_bytes: float, n: int = 4096, k: int = 4096):
        import torch
        import gemm_e2m1_lut_amd as lib
        import synth
        self.lib, self.n, self.k = lib, n, k
        self.name = f"ternary_wl_{n}x{k}"
        per_copy = 4 * (n * k // 4)
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.host = synth.ternary_wl_case(n=n, k=k)
        dev0 = torch.from_numpy(self.host["packed"].view(np.int32)).cuda()
        # rotated copies: the same weights rolled by whole rows (distinct addresses, same statistics)
        self.packed = [torch.roll(dev0, shifts=7 * i, dims=1).contiguous() for i in range(self.copies)]
        self.scale = torch.from_numpy(self.host["scale"]).cuda()
        self.x_re = torch.from_numpy(self.host["x_re"]).cuda()
        self.x_im = torch.from_numpy(self.host["x_im"]).cuda()
        self.y = (torch.empty(n, device="cuda"), torch.empty(n, device="cuda"))
        self.weight_bytes_per_step = float(per_copy + 16 * n)
        self.total_bytes_per_step = float(self.alg_bytes("ternarywl"))
        self.dtype = "f32"
        self.config = {"workload": self.name, "weights": "four 2-bit ternary matrices, 16 per uint32",
                       "activations": "complex fp32 (planar)", "out": "complex fp32 (planar)",
                       "weight_copies_rotated": self.copies}

    def launches(self):
        def fn(i):
            self.lib.ternary_wl_gemv(self.packed[i % self.copies], self.scale, self.x_re, self.x_im,
                                     out=self.y)
        return [("ternarywl", fn)]

    def alg_bytes(self, label):
        # four weight matrices and scale vectors, x_re and x_im, y_re and y_im
        return 4 * (self.n * self.k // 4) + 16 * self.n + 8 * self.k + 8 * self.n

    def cpu_baseline(self, budget_s):
        import oracle
        h = self.host
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.ternary_wl_gemv(h["packed"], h["scale"], h["x_re"], h["x_im"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 2000:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full {self.n} x {self.k} complex layer repeated {reps} times, {el:.1f} s"}


class Gather(Workload):
    def __init__(self, rotate_bytes: float, vocab=200000, hidden=4096, tokens=8192):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib, self.vocab, self.hidden, self.tokens = lib, vocab, hidden, tokens
        self.name = f"nvfp4_embedding_gather_{vocab}x{hidden}_{tokens}ids"
        g = _gen(977)
        self.table = torch.randint(0, 256, (vocab, hidden // 2), dtype=torch.uint8, device="cuda", generator=g)
        u = torch.rand((vocab, hidden // 16), generator=g, device="cuda") * 8 - 4
        self.bscale = torch.exp2(u).to(torch.float8_e4m3fn).view(torch.uint8)
        self.gscale = torch.tensor([0.01], dtype=torch.float32, device="cuda")
        row_bytes = hidden // 2 + hidden // 16
        self.copies = max(2, math.ceil(rotate_bytes / (tokens * row_bytes)))
        self.ids = [torch.randint(0, vocab, (tokens,), device="cuda", generator=g) for _ in range(self.copies)]
        self.out = torch.empty((tokens, hidden), dtype=torch.bfloat16, device="cuda")
        self.weight_bytes_per_step = float(tokens * row_bytes)
        self.total_bytes_per_step = float(self.alg_bytes("gather"))
        self.config = {"workload": self.name, "table": "NVFP4 (E2M1 + E4M3 per 16 + fp32 global)",
                       "out": "bf16", "id_sets_rotated": self.copies}

    def launches(self):
        def fn(i):
            self.lib.nvfp4_embedding_gather(self.table, self.bscale, self.gscale, self.ids[i % self.copies],
                                            out=self.out)
        return [("gather", fn)]

    def alg_bytes(self, label):
        return self.tokens * (self.hidden // 2 + self.hidden // 16 + 8 + 2 * self.hidden)

    def cpu_baseline(self, budget_s):
        import oracle
        sample = 1024
        ids = self.ids[0][:sample].cpu().numpy()
        # the oracle reads only the gathered rows; hand it those rows (same values, bounded memory)
        rows = np.unique(ids)
        remap = np.searchsorted(rows, ids)
        rt = torch_index_rows(self.table, rows)
        rs = torch_index_rows(self.bscale, rows)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.nvfp4_gather(rt, rs, np.float32(0.01), remap)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 2000:
                break
        per = sample * (self.hidden // 2 + self.hidden // 16)
        return {"value": round(per * reps / el / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": f"{sample} of the {self.tokens} ids, repeated {reps} times, {el:.1f} s"}


def torch_index_rows(t, rows: np.ndarray) -> np.ndarray:
    import torch
    return t[torch.from_numpy(rows).to(t.device)].cpu().numpy()


class Decode(Workload):
    def __init__(self, rotate_bytes: float, rows=14336, k=4096):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib, self.rows, self.k = lib, rows, k
        self.name = f"mxfp4_decode_{rows}x{k}"
        g = _gen(31)
        per_copy = rows * k // 2 + rows * k // 32
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.w = [_mxfp4_dev(g, rows, k, 0, 255) for _ in range(self.copies)]
        self.out = torch.empty((rows, k), dtype=torch.bfloat16, device="cuda")
        self.weight_bytes_per_step = float(per_copy)
        self.label = "decode" if rows == 14336 else f"decode_{rows}x{k}"
        self.total_bytes_per_step = float(self.alg_bytes(self.label))
        self.dtype = "u16"
        self.config = {"workload": self.name, "out": "bf16 bit patterns", "weight_copies_rotated": self.copies}

    def launches(self):
        def fn(i):
            p, s = self.w[i % self.copies]
            self.lib.dequant_decode(p, s, out=self.out)
        return [(self.label, fn)]

    def alg_bytes(self, label):
        return self.rows * self.k // 2 + self.rows * self.k // 32 + 2 * self.rows * self.k


class Quantize(Workload):
    """MXFP4 and NVFP4 quantizers on a bf16 matrix of the Llama-8B MLP shape
    14336 x 4096 (weights N(0, 0.02)): one launch of each per step."""

    def __init__(self, rotate_bytes: float, n: int = 14336, k: int = 4096):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib, self.n, self.k = lib, n, k
        self.name = f"quantize_mxfp4_nvfp4_{n}x{k}"
        per_copy = 2 * n * k
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        g = _gen(6161)
        self.x = [(torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
                  for _ in range(self.copies)]
        self.gs = torch.tensor([0.02 * 4 / (6 * 448)], dtype=torch.float32, device="cuda")
        self.mx = (torch.empty(n, k // 2, dtype=torch.uint8, device="cuda"),
                   torch.empty(n, k // 32, dtype=torch.uint8, device="cuda"))
        self.nv = (torch.empty(n, k // 2, dtype=torch.uint8, device="cuda"),
                   torch.empty(n, k // 16, dtype=torch.uint8, device="cuda"))
        self.weight_bytes_per_step = float(2 * per_copy)   # bf16 read by each quantizer
        self.total_bytes_per_step = float(self.alg_bytes("mxquant") + self.alg_bytes("nvquant"))
        self.config = {"workload": self.name, "in": "bf16", "out": "MXFP4 (E8M0 per 32) and NVFP4 (E4M3 per 16)",
                       "weight_copies_rotated": self.copies}

    def launches(self):
        def mx(i):
            self.lib.mxfp4_quantize(self.x[i % self.copies], out=self.mx)

        def nv(i):
            self.lib.nvfp4_quantize(self.x[i % self.copies], self.gs, out=self.nv)
        return [("mxquant", mx), ("nvquant", nv)]

    def alg_bytes(self, label):
        nk = self.n * self.k
        return 2 * nk + nk // 2 + (nk // 32 if label == "mxquant" else nk // 16)

    def cpu_baseline(self, budget_s):
        import oracle
        import synth
        rows = 1024
        x = oracle.bf16_from_f64(synth.rng(6161).standard_normal((rows, self.k)) * 0.02)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.mxfp4_quantize(x)
            oracle.nvfp4_quantize(x, 0.02 * 4 / (6 * 448))
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 2000:
                break
        return {"value": round(2 * 2 * rows * self.k * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"both quantizers on {rows} of the {self.n} rows, repeated {reps} times, {el:.1f} s"}


class Prefill(Workload):
    """MXFP4 weight GEMM for 2048 activation rows (prefill) through the Llama-8B
    MLP matrices 14336 x 4096 and 4096 x 14336, bf16 out: bound by the matrix
    cores, so its roofline is bf16 MFMA."""
    SHAPES = ((14336, 4096), (4096, 14336))
    bound = "mfma"

    def __init__(self, rotate_bytes: float, m: int = 2048):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib, self.m = lib, m
        self.name = f"llama8b_mlp_mxfp4_gemm_m{m}"
        g = _gen(7171)
        # every launch takes longer than the weights take to stream, so rotating copies
        # past the Infinity Cache changes nothing: two copies keep the launch pattern
        self.copies = 2
        self.weights = [[_mxfp4_dev(g, n, k) for n, k in self.SHAPES] for _ in range(self.copies)]
        self.x = [torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16) for _, k in self.SHAPES]
        self.y = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for n, _ in self.SHAPES]
        per_copy = sum(n * k // 2 + n * k // 32 for n, k in self.SHAPES)
        self.weight_bytes_per_step = float(per_copy)
        self.total_bytes_per_step = float(sum(self.alg_bytes(l) for l, _ in self.launches()))
        self.config = {"workload": self.name, "shapes_NxK": [list(s) for s in self.SHAPES], "tokens": m,
                       "weights": "MXFP4 (E2M1 codes + E8M0 per 32)", "activations": "bf16", "out": "bf16",
                       "accumulate": "fp32"}

    def launches(self):
        out = []
        for j, (n, k) in enumerate(self.SHAPES):
            def fn(i, j=j):
                p, s = self.weights[i % self.copies][j]
                self.lib.dequant_gemm(p, s, self.x[j], out=self.y[j])
            out.append((f"gemm_m{self.m}_{n}x{k}", fn))
        return out

    def alg_bytes(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return n * k // 2 + n * k // 32 + self.m * k * 2 + self.m * n * 2

    def alg_flops(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return 2.0 * self.m * n * k

    def cpu_baseline(self, budget_s):
        import oracle
        n, k = self.SHAPES[0]
        p, sc = (t.cpu().numpy() for t in self.weights[0][0])
        xs = self.x[0][:4].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.mxfp4_gemv(p, sc, xs, "bf16")
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 200:
                break
        tflops = 2.0 * 4 * n * k * reps / el / 1e12
        return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
                "sample": f"4 of the {self.m} activation rows through the {n} x {k} matrix, repeated {reps} "
                          f"times, {el:.1f} s, fp64 scalar C"}


class NmSparse(Workload):
    """N:M structured-sparse bf16 weights (kept values + packed in-group
    positions) times one activation row through the Llama-8B MLP matrices
    14336 x 4096 and 4096 x 14336, bf16 out."""
    SHAPES = ((14336, 4096), (4096, 14336))

    def __init__(self, n_keep: int, m: int, rotate_bytes: float, batch: int = 1):
        import torch
        import gemm_e2m1_lut_amd as lib
        self.lib, self.nn, self.mm, self.batch = lib, n_keep, m, batch
        self.name = f"llama8b_mlp_{n_keep}of{m}_sparse_bf16_b{batch}"
        self.bits = 1 if m <= 2 else (m - 1).bit_length()
        g = _gen(8181 + 16 * n_keep + m)
        per_copy = sum(self._wbytes(n, k) for n, k in self.SHAPES)
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.weights = []
        for _ in range(self.copies):
            ws = []
            for n, k in self.SHAPES:
                per_row, words = self._layout(k)
                vals = (torch.randn((n, per_row), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
                # positions uniform over the group (M is a power of two here, so every field is valid)
                meta = torch.randint(-2**31, 2**31 - 1, (n, words), dtype=torch.int32, device="cuda", generator=g)
                ws.append((vals, meta))
            self.weights.append(ws)
        self.x = [torch.randn((batch, k), generator=g, device="cuda").to(torch.bfloat16) for _, k in self.SHAPES]
        self.y = [torch.empty((batch, n), dtype=torch.bfloat16, device="cuda") for n, _ in self.SHAPES]
        self.weight_bytes_per_step = float(per_copy)
        self.total_bytes_per_step = float(sum(self.alg_bytes(l) for l, _ in self.launches()))
        self.config = {"workload": self.name, "shapes_NxK": [list(s) for s in self.SHAPES], "batch": batch,
                       "weights": f"{n_keep}:{m} sparse, bf16 kept values + {self.bits}-bit positions in uint32",
                       "activations": "bf16", "out": "bf16", "accumulate": "fp32",
                       "weight_copies_rotated": self.copies}

    def _layout(self, k):
        per_row = (k // self.mm) * self.nn
        packing = 32 // self.bits
        return per_row, -(-per_row // packing)

    def _wbytes(self, n, k):
        per_row, words = self._layout(k)
        return n * (2 * per_row + 4 * words)

    def launches(self):
        out = []
        for j, (n, k) in enumerate(self.SHAPES):
            def fn(i, j=j):
                v, m = self.weights[i % self.copies][j]
                self.lib.nm_spmm(v, m, self.x[j], self.nn, self.mm, out=self.y[j])
            out.append((f"nm_{self.nn}of{self.mm}_{n}x{k}", fn))
        return out

    def alg_bytes(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return self._wbytes(n, k) + self.batch * k * 2 + self.batch * n * 2

    def alg_flops(self, label):
        n, k = (int(v) for v in label.split("_")[2].split("x"))
        return 2.0 * self.batch * n * self._layout(k)[0]

    def cpu_baseline(self, budget_s):
        import oracle
        import torch
        host = [(v.view(torch.int16).cpu().numpy().view(np.uint16), m.cpu().numpy().view(np.uint32))
                for v, m in self.weights[0]]
        xs = [x.view(torch.int16).cpu().numpy().view(np.uint16) for x in self.x]
        reps, t0 = 0, time.perf_counter()
        while True:
            for (v, m), x, (_, k) in zip(host, xs, self.SHAPES):
                oracle.nm_spmm(v, m, x, k, self.nn, self.mm)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 200:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full step (both MLP shapes, batch {self.batch}) repeated {reps} times, "
                          f"{el:.1f} s, fp64 scalar C with OpenMP over rows"}


class GemvSmall(Workload):
    def __init__(self, rotate_bytes: float):
        import torch
        import gemm_e2m1_lut_amd as lib
        import synth
        self.lib = lib
        self.name = "mxfp4_gemv_256x512_b1"
        c = synth.gemv_small()
        self.p = torch.from_numpy(c["packed"]).cuda()
        self.s = torch.from_numpy(c["scales"]).cuda()
        self.x = torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16).cuda()
        self.y = torch.empty((1, 256), device="cuda")
        # the same buffers, 256 launches per graph: a graph of one launch would time the
        # host's graph launch rather than the kernel
        self.copies = 256
        self.weight_bytes_per_step = 256 * 256 + 256 * 16
        self.total_bytes_per_step = float(self.alg_bytes("gemv_small"))
        self.bound = "latency"
        self.config = {"workload": self.name, "out": "fp32", "note": "fits in L2: launch-latency bound"}

    def launches(self):
        def fn(i):
            self.lib.dequant_gemv(self.p, self.s, self.x, out=self.y)
        return [("gemv_small", fn)]

    def alg_bytes(self, label):
        return 256 * 256 + 256 * 16 + 512 * 2 + 256 * 4

    def cpu_baseline(self, budget_s):
        import oracle
        p, s = self.p.cpu().numpy(), self.s.cpu().numpy()
        x = self.x.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.mxfp4_gemv(p, s, x)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 20000:
                break
        return {"value": round(self.weight_bytes_per_step * reps / el / 1e9, 4), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full 256 x 512 GEMV repeated {reps} times, {el:.1f} s"}


class Moe(Workload):
    def __init__(self, rotate_bytes: float, E=32, H=2880, I=2880, T=256, topk=4):
        import torch
        import gemm_e2m1_lut_amd as lib
        import synth
        self.lib, self.E, self.H, self.I, self.T, self.topk = lib, E, H, I, T, topk
        self.name = f"mxfp4_moe_E{E}_H{H}_I{I}_T{T}_top{topk}"
        g = _gen(5151)
        per_copy = E * (2 * I * H // 2 + 2 * I * H // 32 + H * I // 2 + H * I // 32)
        self.copies = max(2, math.ceil(rotate_bytes / per_copy))
        self.w = []
        for _ in range(self.copies):
            w13, w13s = _mxfp4_dev(g, E * 2 * I, H)
            w2, w2s = _mxfp4_dev(g, E * H, I)
            self.w.append((w13.view(E, 2 * I, H // 2), w13s.view(E, 2 * I, H // 32),
                           w2.view(E, H, I // 2), w2s.view(E, H, I // 32)))
        r = synth.rng(synth.SEED_BASE + 4)
        self.x_host = synth.bf16_normal(r, (T, H))
        ids, wts = synth.router(r, T, E, topk)
        self.ids_host, self.wts_host = ids, wts
        self.x = torch.from_numpy(self.x_host.view(np.int16)).view(torch.bfloat16).cuda()
        self.ids = torch.from_numpy(ids).cuda()
        self.wts = torch.from_numpy(wts).cuda()
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ws = lib.mxfp4_moe_workspace_size(T, H, I, E, topk)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.weight_bytes_per_step = float(per_copy)
        self.total_bytes_per_step = float(self.alg_bytes("moe"))
        self.config = {"workload": self.name, "weights": "MXFP4 W13 [E, 2I, H] + W2 [E, H, I]",
                       "activations": "bf16", "out": "bf16", "mfma": "bf16 16x16x32, fp32 accumulate",
                       "routing": "top-4 of N(0,1) logits, softmax over the selected (input)",
                       "weight_copies_rotated": self.copies, "launch": "entry point (route, gemm1, "
                       "gemm2, combine kernels)"}

    def launches(self):
        def fn(i):
            w13, w13s, w2, w2s = self.w[i % self.copies]
            self.lib.mxfp4_moe_gemm(self.x, w13, w13s, w2, w2s, self.ids, self.wts, out=self.out,
                                    workspace=self.ws)
        return [("moe", fn)]

    def alg_bytes(self, label):
        return self.weight_bytes_per_step + 2 * self.T * self.H * 2 + self.T * self.topk * 8

    def alg_flops(self, label):
        return 2.0 * self.T * self.topk * (2 * self.I * self.H + self.H * self.I)

    def cpu_baseline(self, budget_s):
        import oracle
        sample = 8
        w13, w13s, w2, w2s = (t.cpu().numpy() for t in self.w[0])
        ids, wts = self.ids_host[:sample], self.wts_host[:sample]
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.mxfp4_moe_f64(self.x_host[:sample], w13, w13s, w2, w2s, ids, wts)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 100:
                break
        touched = len(np.unique(ids))
        per_expert = self.weight_bytes_per_step / self.E
        return {"value": round(touched * per_expert * reps / el / 1e9, 3), "unit": "GB/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"{sample} of the {self.T} tokens ({touched} experts' weights decoded), "
                          f"repeated {reps} times, {el:.1f} s"}


# ------------------------------------------------------ platform probe ---
# Reference points measured with the simplest kernels (libe2m1probe.so, built
# beside the library): an empty launch, plain HBM streams of the headline
# launch's size and larger, and a kernel that keeps every matrix core busy.

PROBE_LIB = os.path.join(ROOT, "gemm_e2m1_lut_amd", "probe", "libe2m1probe.so")
_probe = None
# grid sizes of the empty marker launches that `--mark-labels` puts before each launch label
MARK_BASE = 9001


def probe_library():
    global _probe
    if _probe is None:
        import ctypes
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is missing: build with `python -m gemm_e2m1_lut_amd.build`")
        lib = ctypes.CDLL(PROBE_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        for name, res, argt in (("e2m1_probe_empty", i32, [i64, i32, vp]),
                                ("e2m1_probe_stream_grid", i64, [i64, i32]),
                                ("e2m1_probe_stream", i32, [vp, i64, vp, i64, i32, i32, vp]),
                                ("e2m1_probe_mfma", i32, [i64, i32, i32, vp, i64, vp]),
                                ("e2m1_probe_lds", i32, [vp, i64, i32, vp, i64, vp]),
                                ("e2m1_probe_expand", i32, [vp, i64, vp, vp])):
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, argt
        _probe = lib
    return _probe


def _stream_handle():
    import ctypes
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _probe_ok(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def probe_mark(index: int) -> None:
    """An empty launch of MARK_BASE + index workgroups: in a profiler's dispatch list the
    kernels between two marks belong to one launch label."""
    _probe_ok(probe_library().e2m1_probe_empty(MARK_BASE + index, 64, _stream_handle()), "marker")


class EmptyFloor(Workload):
    """Empty kernels, launched back to back from a graph: the per-launch floor."""
    GRIDS = (1, 3808)

    def __init__(self, rotate_bytes: float):
        self.name = "empty_kernel_floor"
        self.copies = 256          # launches of each label per graph
        self.bound = "latency"
        self.metric = "per-launch time of an empty kernel (graph replay, back to back)"
        self.config = {"workload": self.name, "grids": list(self.GRIDS), "block": 64,
                       "launches_per_graph": self.copies}

    def launches(self):
        lib = probe_library()
        out = []
        for grid in self.GRIDS:
            def fn(i, grid=grid):
                _probe_ok(lib.e2m1_probe_empty(grid, 64, _stream_handle()), "empty")
            out.append((f"probe_empty_{grid}x64", fn))
        return out

    def alg_bytes(self, label):
        return 0

    def headline(self, ms_per_step, per_launch):
        return round(1e3 * max(per_launch.values()), 4), "us", False


class HbmStream(Workload):
    """A plain read of `nbytes` from HBM (16-byte non-temporal loads, every load issued
    first), optionally with a small store per wave: the streaming ceiling at that size."""

    STORES = {0: "", 1: "_store", 2: "_store1"}

    def __init__(self, nbytes: int, store: int, rotate_bytes: float, block: int = 64):
        import torch
        self.nbytes, self.store, self.block = nbytes, store, block
        self.name = f"hbm_stream_{nbytes}B" + self.STORES[store]
        self.copies = max(2, math.ceil(rotate_bytes / nbytes))
        g = _gen(777)
        self.bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
                     for _ in range(self.copies)]
        self.grid = int(probe_library().e2m1_probe_stream_grid(nbytes, block))
        if self.grid < 1:
            raise ValueError(f"no stream grid for {nbytes} bytes")
        self.out_words = self.grid * block // 64
        self.out = torch.zeros(self.out_words, dtype=torch.int32, device="cuda")
        self.label = f"probe_stream{self.STORES[store]}_{nbytes}B"
        self.weight_bytes_per_step = float(nbytes)
        self.total_bytes_per_step = float(self.alg_bytes(self.label))
        stored = {0: "none", 1: "4 B per wave", 2: "4 B by the first wave only"}[store]
        self.metric = f"HBM read rate of a plain {nbytes}-byte stream" + ("" if store == 0 else f", store {stored}")
        self.config = {"workload": self.name, "bytes": nbytes, "grid": self.grid, "block": block,
                       "loads_per_lane": "8 x 16 B non-temporal", "store": stored,
                       "buffers_rotated": self.copies, "rotated_MB": round(self.copies * nbytes / 1e6, 1)}

    def launches(self):
        lib = probe_library()

        def fn(i):
            _probe_ok(lib.e2m1_probe_stream(self.bufs[i % self.copies].data_ptr(), self.nbytes,
                                            self.out.data_ptr(), self.out_words, self.block,
                                            self.store, _stream_handle()), "stream")
        return [(self.label, fn)]

    def alg_bytes(self, label):
        return self.nbytes + {0: 0, 1: 4 * self.out_words, 2: 4}[self.store]

    def headline(self, ms_per_step, per_launch):
        return round(self.nbytes / (per_launch[self.label] * 1e-3) / 1e9, 2), "GB/s", True


class ExpandStream(Workload):
    """Reads `src_bytes` and writes four times as many (16 bytes in, 64 out per chunk, the
    byte ratio of a 4-bit code to its bf16 decode): the streaming reference of the
    write-heavy kernels at their sizes."""

    def __init__(self, src_bytes: int, rotate_bytes: float):
        import torch
        self.src_bytes = src_bytes
        self.name = f"hbm_expand_{src_bytes}B"
        self.label = f"probe_expand_{src_bytes}B"
        self.copies = max(2, math.ceil(rotate_bytes / (5 * src_bytes)))
        g = _gen(778)
        self.src = [torch.randint(0, 256, (src_bytes,), dtype=torch.uint8, device="cuda", generator=g)
                    for _ in range(self.copies)]
        self.dst = [torch.empty(4 * src_bytes, dtype=torch.uint8, device="cuda") for _ in range(self.copies)]
        self.weight_bytes_per_step = float(src_bytes)
        self.total_bytes_per_step = float(self.alg_bytes(self.label))
        self.metric = f"HBM rate of a stream reading {src_bytes} bytes and writing {4 * src_bytes}"
        self.config = {"workload": self.name, "read_bytes": src_bytes, "write_bytes": 4 * src_bytes,
                       "per_chunk": "16 B non-temporal load, 4 x 16 B non-temporal stores",
                       "buffers_rotated": self.copies}

    def launches(self):
        lib = probe_library()

        def fn(i):
            _probe_ok(lib.e2m1_probe_expand(self.src[i % self.copies].data_ptr(), self.src_bytes,
                                            self.dst[i % self.copies].data_ptr(), _stream_handle()), "expand")
        return [(self.label, fn)]

    def alg_bytes(self, label):
        return 5 * self.src_bytes

    def headline(self, ms_per_step, per_launch):
        return round(self.alg_bytes("") / (per_launch[self.label] * 1e-3) / 1e9, 2), "GB/s", True


class MfmaPeak(Workload):
    """Four independent bf16 MFMA chains per wave, two waves per SIMD: the matrix-core
    rate a kernel can reach with one instruction shape (form 32: v_mfma_f32_32x32x16_bf16,
    form 16: v_mfma_f32_16x16x32_bf16), and the reading of the MFMA-busy counter for a
    kernel that keeps the matrix cores saturated."""
    GRID, ITERS = 512, 2048

    def __init__(self, rotate_bytes: float, form: int = 32):
        import torch
        self.form = form
        self.shape = "32x32x16" if form == 32 else "16x16x32"
        self.label = f"probe_mfma_{self.shape}"
        self.name = "mfma_bf16_peak" + ("" if form == 32 else "_16x16x32")
        self.copies = 4
        self.bound = "mfma"
        self.out = torch.zeros(self.GRID * 256, dtype=torch.float32, device="cuda")
        self.metric = f"bf16 MFMA rate of a kernel of back-to-back independent {self.shape} MFMAs"
        self.config = {"workload": self.name, "grid": self.GRID, "block": 256, "iters": self.ITERS,
                       "chains_per_wave": 4, "instruction": f"v_mfma_f32_{self.shape}_bf16"}

    def launches(self):
        lib = probe_library()

        def fn(i):
            _probe_ok(lib.e2m1_probe_mfma(self.GRID, self.ITERS, self.form, self.out.data_ptr(),
                                          self.out.numel(), _stream_handle()), "mfma")
        return [(self.label, fn)]

    def alg_bytes(self, label):
        return 0

    def alg_flops(self, label):
        return float(self.GRID * 4 * self.ITERS * 4 * (32768 if self.form == 32 else 16384))

    def headline(self, ms_per_step, per_launch):
        return round(self.alg_flops("") / (per_launch[self.label] * 1e-3) / 1e12, 1), "TFLOP/s", True


def lds_pattern(name: str, lane: int) -> int:
    """16-byte LDS slot read by `lane` (0..63) in the LDS read-rate probe. r = lane % 16 and
    g = lane // 16 are the MFMA operand layout's row and lane group."""
    r, g = lane % 16, lane // 16
    return {
        "contiguous": lane,                                  # 1 KB in lane order
        "rows33_shift4": 33 * r + 4 * g,                     # padded 528-byte rows, groups 64 bytes apart
        "rows9_shift1": 9 * r + g,                           # padded 144-byte rows, groups 16 bytes apart
        "rows8_xor": 8 * r + (g ^ ((r >> 1) & 7)),           # 128-byte rows, block index XOR row / 2
        "chunk_major": 256 * g + r,                          # 16 rows contiguous per group, groups 4 KB apart
        "pitch256": 16 * lane,                               # every lane in one bank group
    }[name]


LDS_PATTERNS = ("contiguous", "rows33_shift4", "rows9_shift1", "rows8_xor", "chunk_major", "pitch256")


class LdsRead(Workload):
    """LDS read rate of one lane -> 16-byte slot pattern: one 512-thread workgroup per
    compute unit, every wave reading the pattern with back-to-back ds_read_b128."""
    GRID_PER_CU, ITERS = 1, 256

    def __init__(self, rotate_bytes: float, pattern: str):
        import torch
        self.pattern = pattern
        self.name = f"lds_read_{pattern}"
        self.label = f"probe_lds_{pattern}"
        self.copies = 4
        self.bound = "lds"
        self.grid = self.GRID_PER_CU * torch.cuda.get_device_properties(0).multi_processor_count
        table = [lds_pattern(pattern, l) for l in range(64)]
        self.table = torch.tensor(table, dtype=torch.int32, device="cuda")
        self.out = torch.zeros(self.grid * 512, dtype=torch.int32, device="cuda")
        self.metric = f"LDS read rate, ds_read_b128, pattern {pattern}, eight waves per compute unit"
        self.config = {"workload": self.name, "grid": self.grid, "block": 512, "iters": self.ITERS,
                       "reads_per_lane": 8 * self.ITERS, "slots": table}

    def launches(self):
        lib = probe_library()

        def fn(i):
            _probe_ok(lib.e2m1_probe_lds(self.table.data_ptr(), self.grid, self.ITERS, self.out.data_ptr(),
                                         self.out.numel(), _stream_handle()), "lds")
        return [(self.label, fn)]

    def alg_bytes(self, label):   # HBM bytes: none (the array lives in LDS)
        return 0

    def lds_bytes(self) -> float:
        return float(self.grid * 512 * 16 * 8 * self.ITERS)

    def headline(self, ms_per_step, per_launch):
        return round(self.lds_bytes() / (per_launch[self.label] * 1e-3) / 1e12, 2), "TB/s", True


HEADLINE_BYTES = 14336 * 4096 // 2 + 14336 * 4096 // 32   # one batch-1 MLP GEMV launch's weights
TERNARY_BYTES = 4096 * 4096 // 4                            # the 4096 x 4096 ternary matrix (2 bits a weight)

WORKLOADS = {
    "floor": EmptyFloor,
    "stream_31mb": lambda rb: HbmStream(HEADLINE_BYTES, 0, rb),
    "stream_31mb_store": lambda rb: HbmStream(HEADLINE_BYTES, 1, rb),
    "stream_31mb_store1": lambda rb: HbmStream(HEADLINE_BYTES, 2, rb),
    "stream_4mb_store": lambda rb: HbmStream(TERNARY_BYTES, 1, rb),
    "stream_17mb_store": lambda rb: HbmStream(4 * TERNARY_BYTES, 1, rb),   # the widely-linear layer's four matrices
    "stream_128mb": lambda rb: HbmStream(128 << 20, 0, rb),
    "stream_512mb": lambda rb: HbmStream(512 << 20, 0, rb),
    "expand_29mb": lambda rb: ExpandStream(14336 * 4096 // 2, rb),
    "expand_17mb": lambda rb: ExpandStream(8192 * 4096 // 2, rb),
    "mfma_peak": MfmaPeak,
    "mfma_peak_16x16x32": lambda rb: MfmaPeak(rb, 16),
    "moe": Moe,
    "mlp_b1": lambda rb: GemvMLP(1, rb),
    "mlp_b1_grouped": GemvMLPGrouped,
    "mlp_b2": lambda rb: GemvMLP(2, rb),
    "mlp_b4": lambda rb: GemvMLP(4, rb),
    "mlp_b8": lambda rb: GemvMLP(8, rb),
    "mlp_b16": lambda rb: GemvMLP(16, rb),
    "ternary": Ternary,
    "ternary_wl": TernaryWL,
    "ternary_b1": lambda rb: TernaryBatch(1, rb),
    "ternary_b2": lambda rb: TernaryBatch(2, rb),
    "ternary_b4": lambda rb: TernaryBatch(4, rb),
    "ternary_b6": lambda rb: TernaryBatch(6, rb),
    "ternary_b8": lambda rb: TernaryBatch(8, rb),
    "ternary_b16": lambda rb: TernaryBatch(16, rb),
    "gather": Gather,
    "decode": Decode,
    "decode_8192": lambda rb: Decode(rb, rows=8192),
    "quantize": Quantize,
    "prefill": Prefill,
    "nm_2of4": lambda rb: NmSparse(2, 4, rb),
    "nm_4of8": lambda rb: NmSparse(4, 8, rb),
    "gemv_small": GemvSmall,
}
WORKLOADS.update({f"lds_{p}": (lambda p: lambda rb: LdsRead(rb, p))(p) for p in LDS_PATTERNS})


# ---------------------------------------------------------------- timing ---
#
# Steps are captured into a HIP graph (torch.cuda.CUDAGraph) and replayed, so
# the timed region contains only the kernels: an eager Python launch costs
# more host time than these kernels take on the GPU. One graph holds one step
# per weight copy (every copy once); the per-kernel graphs hold one launch of
# a single kernel per copy.


def _capture(fns, copies: int, offset: int):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(copies):
                for fn in fns:
                    fn(offset + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _time_replays(g, replays: int) -> float:
    """Milliseconds for `replays` graph replays (events on torch's current stream)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def timed_steps(launches, copies: int, steps: int, warmup: int) -> tuple[float, int]:
    """(milliseconds per step, steps actually timed): whole steps, graph-replayed."""
    g = _capture([fn for _, fn in launches], copies, 0)
    reps = max(1, math.ceil(steps / copies))
    for _ in range(max(1, math.ceil(warmup / copies))):
        g.replay()
    ms = _time_replays(g, reps)
    return ms / (reps * copies), reps * copies


def per_launch_ms(launches, copies: int, steps: int) -> dict:
    """Average duration of each launch label: a graph of that kernel alone, replayed."""
    out = {}
    for label, fn in launches:
        g = _capture([fn], copies, 0)
        reps = max(1, math.ceil(steps / copies))
        out[label] = _time_replays(g, reps) / (reps * copies)
    return out


def copy_calibration(mb: int) -> None:
    """A plain elementwise copy (read mb MiB, write mb MiB), run three times: a kernel of
    known traffic that checks the byte counts taken from the memory request counters."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def traffic_from_profile(label: str) -> dict | None:
    """Measured HBM bytes per launch from a committed counter summary, if the kernels
    have not changed since it was taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    entry = data.get(label)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(label):
        return None
    return entry


def cpu_description() -> dict:
    """What identifies the host CPU: /proc/cpuinfo's fields for the first processor (model name,
    vendor, family, model, stepping, cache size, clock), the number of logical processors, the
    CPUs this process may run on, and the L2/L3 sizes from sysfs."""
    info: dict = {}
    keys = ("model name", "vendor_id", "cpu family", "model", "stepping", "cache size", "cpu MHz",
            "cpu cores", "siblings")
    try:
        with open("/proc/cpuinfo") as fh:
            text = fh.read()
        first = text.split("\n\n")[0]
        for line in first.splitlines():
            k, _, v = line.partition(":")
            k = k.strip()
            if k in keys and k not in info:
                info[k] = v.strip()
        info["logical_processors"] = text.count("processor\t:")
    except OSError:
        pass
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    cache = "/sys/devices/system/cpu/cpu0/cache"
    for idx in range(8):
        d = os.path.join(cache, f"index{idx}")
        try:
            with open(os.path.join(d, "level")) as fh:
                level = fh.read().strip()
            with open(os.path.join(d, "type")) as fh:
                kind = fh.read().strip()
            with open(os.path.join(d, "size")) as fh:
                size = fh.read().strip()
        except OSError:
            continue
        if kind in ("Unified", "Data"):
            info[f"L{level}{'d' if kind == 'Data' else ''}"] = size
    return info


def run_cpu_baseline(wl, budget_s: float, budget_1core_s: float) -> dict | None:
    """The oracle on this host: on all its OpenMP threads, then on one."""
    import oracle
    cpu = wl.cpu_baseline(budget_s)
    if cpu is None:
        return None
    n0 = oracle.threads()
    try:
        oracle.set_threads(1)
        one = wl.cpu_baseline(budget_1core_s)
    finally:
        oracle.set_threads(n0)
    cpu["single_core"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
    desc = cpu_description()
    cpu["cpu_model"] = desc.get("model name", "unknown")
    cpu["cpu"] = desc
    cpu["build"] = "gcc " + " ".join(oracle.CFLAGS)
    return cpu


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_b1", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate-mb", type=float, default=600.0,
                    help="weight bytes cycled through per pass (> 256 MB Infinity Cache)")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0, help="run a plain copy of this size first "
                    "(counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--mark-labels", action="store_true",
                    help="before the warmup, run each launch label once after an empty marker launch of "
                         f"{MARK_BASE} + index workgroups (for attributing profiler records to labels); "
                         f"with --copy-mb, the copies sit between two marks of {MARK_BASE - 1}")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; its value is that GPU's throughput)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    import gemm_e2m1_lut_amd as lib
    lib.load_library()
    torch.cuda.set_device(0)

    if args.copy_mb:
        if args.mark_labels:
            probe_mark(-1)
        copy_calibration(args.copy_mb)
        if args.mark_labels:
            probe_mark(-1)

    wl = WORKLOADS[args.workload](args.rotate_mb * 1e6)
    launches = wl.launches()
    if args.mark_labels:
        torch.cuda.synchronize()
        for j, (_, fn) in enumerate(launches):
            probe_mark(j)
            fn(0)
        probe_mark(len(launches))
        torch.cuda.synchronize()
        print(json.dumps({"label_marks": {label: MARK_BASE + j for j, (label, _) in enumerate(launches)},
                          "end_mark": MARK_BASE + len(launches)}), file=sys.stderr, flush=True)
    for i in range(max(2, wl.copies)):          # eager warmup: fills the library's launch caches
        for _, fn in launches:
            fn(i)
    torch.cuda.synchronize()

    ms_per_step, steps_timed = timed_steps(launches, wl.copies, args.steps, args.warmup)
    per_launch = per_launch_ms(launches, wl.copies, args.steps)

    value = wl.weight_bytes_per_step / (ms_per_step * 1e-3) / 1e9
    unit, higher = "GB/s", True
    if wl.metric is not None:
        value, unit, higher = wl.headline(ms_per_step, per_launch)
    pct_hbm = wl.total_bytes_per_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS * 100.0

    kernels = []
    for label, _ in launches:
        ms = per_launch[label]
        kernels.append({"label": label, "avg_us": round(ms * 1e3, 3),
                        "alg_bytes": int(wl.alg_bytes(label)),
                        "GBps": round(wl.alg_bytes(label) / (ms * 1e-3) / 1e9, 1)})
    dom = max(kernels, key=lambda k: k["avg_us"])
    achieved = dom["GBps"]
    traffic = traffic_from_profile(dom["label"])
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": dom["label"]}
    if getattr(wl, "bound", "hbm") == "mfma":
        tflops = wl.alg_flops(dom["label"]) / (dom["avg_us"] * 1e-6) / 1e12
        roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)})
    elif getattr(wl, "bound", "hbm") == "lds":   # no published per-CU LDS figure to divide by
        roofline.update({"bound": "lds", "achieved": round(wl.lds_bytes() / (dom["avg_us"] * 1e-6) / 1e12, 2),
                         "peak": None, "unit": "TB/s", "frac": None})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(wl, args.cpu_budget_s, args.cpu_budget_s)

    line = {
        "metric": wl.metric or METRIC,
        "value": round(value, 4 if unit == "us" else 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": higher,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": wl.config,
        "pct_hbm_peak": round(pct_hbm, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    flops = wl.alg_flops(dom["label"])
    if flops > 0 and wl.bound == "hbm" and args.workload in ("moe", "mlp_b4", "mlp_b16"):
        tflops = flops / (dom["avg_us"] * 1e-6) / 1e12
        line["mfma"] = {"achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": flops}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
