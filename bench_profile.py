#!/usr/bin/env python3
"""rocprofv3 profiles of bench.py workloads: kernel durations and hardware counters.

    python3 bench_profile.py --workload mlp_b1 [--workload moe ...] --out gpurun_out/prof [--write]
    python3 bench_profile.py --workload mlp_b1 --out gpurun_out/prof --parse-only [--write]

For each workload this runs, one child process at a time and each under its own
time limit (this process never touches the GPU):

  bench   python3 bench.py --workload W --no-cpu-baseline               (no profiler: event timing)
  trace   rocprofv3 --kernel-trace --stats -- python3 bench.py --workload W --mark-labels ...
  reads   rocprofv3 --pmc TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B TCC_EA0_RDREQ_128B TCC_EA0_RDREQ -- ...
  writes  rocprofv3 --pmc TCC_EA0_WRREQ TCC_EA0_WRREQ_64B TCC_HIT TCC_MISS -- ...
  busy    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU
                          SQ_WAIT_INST_ANY SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT
                          SQ_WAVE_CYCLES GRBM_GUI_ACTIVE -- ...

bench.py's --mark-labels puts an empty launch of a known grid before each launch
label's first call, so every profiler record is attributed to the label whose
kernels (name, grid, workgroup) appeared after that label's mark. The counter
passes also run three plain 256 MiB copies between two marks first: a kernel of
known traffic that checks the byte arithmetic.

HBM bytes are taken from the L2's memory-side request counters by request size:
read = 32 R32 + 64 R64 + 128 R128 and write = 64 W64 + 32 (W - W64), per
dispatch, with the copy's measured/known ratio reported (and applied as the
calibration factor). Unit busy fractions are ratios to GRBM_GUI_ACTIVE (GPU busy
cycles, which rocprofv3 reports summed over the 8 XCDs).

The summary goes to stdout and OUT/W/summary.txt; --write also stores it as
profiles/<name>.txt and records each label's measured bytes per launch in
profiles/traffic.json (keyed by bench.py's kernel source hash).
"""
from __future__ import annotations

import argparse
import csv
import glob
import gzip
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
BENCH = os.path.join(ROOT, "bench.py")
PROFILES = os.path.join(ROOT, "profiles")
MARK_BASE = 9001          # bench.py's marker grids: MARK_BASE + label index; MARK_BASE - 1 brackets the copies
COPY_MIB = 256
XCDS = 8
SIMDS = 1024              # 256 CUs x 4 SIMDs
CUS = 256

PASSES = {
    "reads": ["TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B", "TCC_EA0_RDREQ"],
    "writes": ["TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B", "TCC_HIT", "TCC_MISS"],
    "busy": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY",
             "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
}

# profile file name per workload
PROFILE_NAMES = {
    "mlp_b1": "gemv_b1_llama8b_mlp", "mlp_b1_grouped": "gemv_b1_grouped_llama8b_mlp", "mlp_b2": "gemv_b2_llama8b_mlp", "mlp_b4": "gemv_b4_llama8b_mlp",
    "mlp_b8": "gemv_b8_llama8b_mlp",
    "mlp_b16": "gemv_b16_llama8b_mlp", "gemv_small": "gemv_b1_256x512",
    "ternary": "ternary_gemv_4096x4096", "ternary_wl": "ternary_wl_4096x4096",
    "ternary_b1": "ternary_gemm_b1_4096x4096", "ternary_b2": "ternary_gemm_b2_4096x4096",
    "ternary_b4": "ternary_gemm_b4_4096x4096", "ternary_b6": "ternary_gemm_b6_4096x4096",
    "ternary_b8": "ternary_gemm_b8_4096x4096",
    "ternary_b16": "ternary_gemm_b16_4096x4096",
    "gather": "nvfp4_gather_200000x4096_8192ids", "decode": "mxfp4_decode_14336x4096",
    "decode_8192": "mxfp4_decode_8192x4096",
    "quantize": "quantize_mxfp4_nvfp4_14336x4096", "prefill": "gemm_m2048_llama8b_mlp",
    "nm_2of4": "nm_2of4_b1_llama8b_mlp", "nm_4of8": "nm_4of8_b1_llama8b_mlp",
    "moe": "moe_E32_H2880_I2880_T256_top4",
    "floor": "platform_empty_kernel", "stream_31mb": "platform_hbm_stream_31mb",
    "stream_31mb_store": "platform_hbm_stream_31mb_store", "stream_31mb_store1": "platform_hbm_stream_31mb_store1",
    "stream_4mb_store": "platform_hbm_stream_4mb_store", "stream_17mb_store": "platform_hbm_stream_17mb_store", "stream_128mb": "platform_hbm_stream_128mb",
    "stream_512mb": "platform_hbm_stream_512mb", "mfma_peak": "platform_mfma_bf16",
    "mfma_peak_16x16x32": "platform_mfma_bf16_16x16x32",
    "expand_29mb": "platform_hbm_expand_29mb_to_117mb", "expand_17mb": "platform_hbm_expand_17mb_to_67mb",
    **{f"lds_{p}": f"platform_lds_read_{p}" for p in ("contiguous", "rows33_shift4", "rows9_shift1", "rows8_xor",
                                                      "chunk_major", "pitch256")},
}


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


# ------------------------------------------------------------------ running ---

def bench_args(workload: str, pmc: bool, steps: int) -> list[str]:
    a = [sys.executable, BENCH, "--workload", workload, "--no-cpu-baseline", "--mark-labels"]
    if pmc:
        a += ["--steps", "20", "--warmup", "2", "--copy-mb", str(COPY_MIB)]
    else:
        a += ["--steps", str(steps)]
    return a


def commands(workload: str, out: str, steps: int, passes: list[str]) -> list[tuple[str, list[str]]]:
    d = os.path.join(out, workload)
    cmds = []
    if "bench" in passes:
        cmds.append(("bench", ["timeout", "-k", "10", "300", sys.executable, BENCH, "--workload", workload,
                               "--no-cpu-baseline"]))
    if "trace" in passes:
        cmds.append(("trace", ["timeout", "-k", "10", "300", "rocprofv3", "--kernel-trace", "--stats",
                               "--output-format", "csv", "-d", os.path.join(d, "trace"), "-o", "run", "--",
                               *bench_args(workload, False, steps)]))
    for name, counters in PASSES.items():
        if name in passes:
            cmds.append((name, ["timeout", "-s", "KILL", "150", "rocprofv3", "--pmc", *counters,
                                "--output-format", "csv", "-d", os.path.join(d, name), "-o", "run", "--",
                                *bench_args(workload, True, steps)]))
    return cmds


def run_all(workload: str, out: str, steps: int, passes: list[str]) -> bool:
    d = os.path.join(out, workload)
    os.makedirs(d, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    with open(os.path.join(d, "commands.txt"), "w") as fh:
        for name, cmd in commands(workload, out, steps, passes):
            fh.write(f"{name}: cd /tmp && TMPDIR=/tmp {' '.join(cmd).replace(ROOT, '<repo>')}\n")
    for name, cmd in commands(workload, out, steps, passes):
        log(f"{workload}: {name} ...")
        t0 = time.time()
        with open(os.path.join(d, f"{name}.stdout"), "w") as so, open(os.path.join(d, f"{name}.stderr"), "w") as se:
            rc = subprocess.call(cmd, cwd="/tmp", env=env, stdout=so, stderr=se)
        printed = _json_line(os.path.join(d, f"{name}.stdout")) is not None
        log(f"{workload}: {name} exit {rc} after {time.time() - t0:.1f} s" + ("" if printed else ", no result line"))
        # rocprofv3 itself may end with SIGSEGV after the program has finished and its files are whole
        if rc != 0 and not (rc in (139, -11) and name != "bench" and printed):
            log(f"{workload}: stopping after {name} (exit {rc}); see {d}/{name}.stderr")
            return False
    _compress(d)
    return True


def _compress(d: str) -> None:
    """gzip the profiler's CSV files (the records of a workload run to tens of MB)."""
    for path in glob.glob(os.path.join(d, "**", "*.csv"), recursive=True):
        with open(path, "rb") as src, gzip.open(path + ".gz", "wb", compresslevel=6) as dst:
            dst.write(src.read())
        os.remove(path)


# ------------------------------------------------------------------ parsing ---

def _json_line(path: str) -> dict | None:
    if not os.path.exists(path):
        return None
    for line in reversed(open(path).read().splitlines()):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return None


def short_name(kernel: str) -> str:
    """Kernel function name with its template arguments, without namespaces or parameters."""
    k = kernel.strip()
    if k.startswith("void "):
        k = k[5:]
    depth, cut = 0, len(k)
    for i, ch in enumerate(k):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not k[:i].endswith("(anonymous namespace"):
            if k[i:].startswith("(anonymous namespace)"):
                continue
            cut = i
            break
    k = k[:cut]
    depth, last = 0, 0
    for i, ch in enumerate(k):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and k[i:i + 2] == "::":
            last = i + 2
    return k[last:]


def _size(row: dict, key: str) -> int:
    if key in row and row[key] not in ("", None):
        return int(float(row[key]))
    return int(float(row.get(key + "_X", 1))) * int(float(row.get(key + "_Y", 1))) * int(float(row.get(key + "_Z", 1)))


def _find(d: str, suffix: str) -> str | None:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True) +
                  glob.glob(os.path.join(d, "**", f"*{suffix}.gz"), recursive=True))
    return hits[0] if hits else None


def _open_text(path: str):
    return gzip.open(path, "rt") if path.endswith(".gz") else open(path)


def dispatches(path: str) -> list[dict]:
    """One record per dispatch: id, kernel short name, grid (work-items), workgroup, and
    either its duration (kernel trace) or its counter values (counter collection)."""
    by_id: dict = {}
    with _open_text(path) as fh:
        for r in csv.DictReader(fh):
            did = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or len(by_id))
            rec = by_id.get(did)
            if rec is None:
                rec = {"id": did, "kernel": short_name(r["Kernel_Name"]), "grid": _size(r, "Grid_Size"),
                       "wg": _size(r, "Workgroup_Size"), "counters": {}}
                if "Start_Timestamp" in r and "End_Timestamp" in r:
                    rec["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    rec["start"] = int(r["Start_Timestamp"])
                by_id[did] = rec
            if "Counter_Name" in r:
                rec["counters"][r["Counter_Name"]] = rec["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [by_id[k] for k in sorted(by_id)]


def _mark_index(rec: dict) -> int | None:
    if "probe_empty_kernel" not in rec["kernel"] or rec["wg"] != 64:
        return None
    for g in (rec["grid"] // 64, rec["grid"]):
        if MARK_BASE - 1 <= g < MARK_BASE + 64:
            return g - MARK_BASE
    return None


def attribute(recs: list[dict], labels: list[str]) -> tuple[dict, list[dict]]:
    """(label -> list of records, copy records). A record belongs to a label when its
    (kernel, grid, workgroup) appeared between that label's mark and the next."""
    sig_label: dict = {}
    copies: list[dict] = []
    current, in_copy = None, False
    for r in recs:
        m = _mark_index(r)
        if m is not None:
            if m == -1:
                in_copy = not in_copy
                current = None
            else:
                current = m if m < len(labels) else None
            continue
        if in_copy:
            copies.append(r)
        elif current is not None:
            sig_label.setdefault((r["kernel"], r["grid"], r["wg"]), set()).add(labels[current])
    out: dict = {label: [] for label in labels}
    for r in recs:
        if _mark_index(r) is not None:
            continue
        for label in sig_label.get((r["kernel"], r["grid"], r["wg"]), ()):
            out[label].append(r)
    return out, copies


def _labels_from(d: str) -> list[str]:
    for name in ("bench", "trace", "reads", "writes", "busy"):
        j = _json_line(os.path.join(d, f"{name}.stdout"))
        if j:
            return [k["label"] for k in j["kernels"]]
    return []


def _by_signature(recs: list[dict]) -> dict:
    sig: dict = {}
    for r in recs:
        sig.setdefault((r["kernel"], r["grid"], r["wg"]), []).append(r)
    return sig


def _pct(v: list[float], q: float) -> float:
    v = sorted(v)
    if not v:
        return float("nan")
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def summarize(workload: str, out: str) -> tuple[str, dict]:
    d = os.path.join(out, workload)
    labels = _labels_from(d)
    bench = _json_line(os.path.join(d, "bench.stdout"))
    alg = {k["label"]: k["alg_bytes"] for k in bench["kernels"]} if bench else {}
    lines = [f"workload {workload}: {bench['config'] if bench else ''}", ""]
    records: dict = {}

    # durations
    tr = _find(os.path.join(d, "trace"), "kernel_trace.csv")
    if tr:
        per_label, _ = attribute(dispatches(tr), labels)
        lines.append("Kernel durations (rocprofv3 kernel trace; every launch of the run: warmup, the timed")
        lines.append("graph replays and the per-launch timing graphs):")
        lines.append("")
        lines.append(f"  {'label':28s} {'kernel':44s} {'grid':>9s} {'wg':>4s} {'calls':>6s} {'mean':>8s} "
                     f"{'median':>8s} {'p10':>8s} {'p90':>8s} {'min':>8s} {'max':>8s}")
        for label in labels:
            for (k, g, w), rs in _by_signature(per_label[label]).items():
                us = [r["us"] for r in rs]
                lines.append(f"  {label:28s} {k[:44]:44s} {g:9d} {w:4d} {len(us):6d} {statistics.mean(us):8.3f} "
                             f"{statistics.median(us):8.3f} {_pct(us, .1):8.3f} {_pct(us, .9):8.3f} {min(us):8.3f} "
                             f"{max(us):8.3f}")
                records.setdefault(label, {}).setdefault("durations", {})[f"{k} grid {g} wg {w}"] = {
                    "calls": len(us), "mean_us": round(statistics.mean(us), 3),
                    "median_us": round(statistics.median(us), 3), "p10_us": round(_pct(us, .1), 3),
                    "p90_us": round(_pct(us, .9), 3), "min_us": round(min(us), 3)}
        lines.append("")
    if bench:
        lines.append("bench.py without the profiler (HIP events around graph replays of one launch label):")
        lines.append("")
        for k in bench["kernels"]:
            lines.append(f"  {k['label']:28s} {k['avg_us']:9.3f} us   algorithmic {k['alg_bytes']:>11d} B   "
                         f"{k['GBps']:8.1f} GB/s")
        lines.append(f"  step {bench['ms_per_step'] * 1e3:.3f} us   value {bench['value']} {bench['unit']}   "
                     f"roofline frac {bench['roofline']['frac']}")
        lines.append("")

    # counters
    per_pass = {}
    copy_check = {}
    for name in PASSES:
        f = _find(os.path.join(d, name), "counter_collection.csv")
        if f:
            per_label, copies = attribute(dispatches(f), labels)
            per_pass[name] = per_label
            if copies:
                copy_check[name] = copies
    fr = fw = None
    if "reads" in copy_check:
        big = [r for r in copy_check["reads"] if r["counters"].get("TCC_EA0_RDREQ", 0) > 1e6]
        if big:
            rb = statistics.median(_read_bytes(r["counters"]) for r in big)
            fr = COPY_MIB * 2 ** 20 / rb
    if "writes" in copy_check:
        big = [r for r in copy_check["writes"] if r["counters"].get("TCC_EA0_WRREQ", 0) > 1e6]
        if big:
            wb = statistics.median(_write_bytes(r["counters"]) for r in big)
            fw = COPY_MIB * 2 ** 20 / wb
    if "reads" in per_pass or "writes" in per_pass:
        lines.append("HBM traffic per launch (median over the label's dispatches; read = 32 R32 + 64 R64 + 128 R128,")
        lines.append("write = 64 W64 + 32 (W - W64), from TCC_EA0_RDREQ_{32B,64B,128B} and TCC_EA0_WRREQ{,_64B};")
        lines.append(f"the {COPY_MIB} MiB copy reads as known/measured = "
                     f"{'%.4f' % fr if fr else 'n/a'} (read), {'%.4f' % fw if fw else 'n/a'} (write),")
        lines.append("applied as calibration factors):")
        lines.append("")
        lines.append(f"  {'label':28s} {'kernel':44s} {'R32':>9s} {'R64':>9s} {'R128':>9s} {'RDREQ':>9s} "
                     f"{'read MB':>9s} {'write MB':>9s} {'L2 hit':>7s}")
        for label in labels:
            tot_r = tot_w = 0.0
            sigs_r = _by_signature(per_pass.get("reads", {}).get(label, []))
            sigs_w = _by_signature(per_pass.get("writes", {}).get(label, []))
            for sig in sorted(set(sigs_r) | set(sigs_w)):
                k, g, w = sig
                cr = _median_counters(sigs_r.get(sig, []))
                cw = _median_counters(sigs_w.get(sig, []))
                rb = _read_bytes(cr) * (fr or 1.0) if cr else 0.0
                wb = _write_bytes(cw) * (fw or 1.0) if cw else 0.0
                tot_r += rb
                tot_w += wb
                hit = cw.get("TCC_HIT", 0) / max(1.0, cw.get("TCC_HIT", 0) + cw.get("TCC_MISS", 0)) if cw else float("nan")
                lines.append(f"  {label:28s} {k[:44]:44s} {cr.get('TCC_EA0_RDREQ_32B', 0):9.0f} "
                             f"{cr.get('TCC_EA0_RDREQ_64B', 0):9.0f} {cr.get('TCC_EA0_RDREQ_128B', 0):9.0f} "
                             f"{cr.get('TCC_EA0_RDREQ', 0):9.0f} {rb / 1e6:9.3f} {wb / 1e6:9.3f} {hit:7.3f}")
            rec = records.setdefault(label, {})
            rec.update({"read_bytes": int(tot_r), "write_bytes": int(tot_w), "bytes_per_launch": int(tot_r + tot_w)})
            if label in alg and alg[label]:
                rec["alg_bytes"] = alg[label]
        lines.append("")
        for label in labels:
            rec = records.get(label, {})
            if rec.get("alg_bytes"):
                lines.append(f"  {label}: measured {rec['bytes_per_launch'] / 1e6:.3f} MB per launch vs algorithmic "
                             f"{rec['alg_bytes'] / 1e6:.3f} MB ({rec['bytes_per_launch'] / rec['alg_bytes']:.3f}x)")
        lines.append("")
        for rec in records.values():
            rec["calibration"] = {"read": round(fr, 4) if fr else None, "write": round(fw, 4) if fw else None}

    if "busy" in per_pass:
        lines.append("Unit activity (median per dispatch; GUI = GRBM_GUI_ACTIVE summed over the 8 XCDs, so")
        lines.append(f"GUI/8 = busy cycles; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI/8 x {SIMDS} SIMDs),")
        lines.append(f"VALU / LDS active = SQ_ACTIVE_INST_{{VALU,LDS}} / SQ_BUSY_CU_CYCLES, wait = SQ_WAIT_INST_ANY /")
        lines.append("SQ_WAVE_CYCLES, bank conflicts per LDS instruction):")
        lines.append("")
        lines.append(f"  {'label':28s} {'kernel':44s} {'GUI/8':>9s} {'MFMAbusy':>9s} {'VALUact':>8s} {'LDSact':>8s} "
                     f"{'wait':>6s} {'bc/LDS':>7s}  raw")
        for label in labels:
            for (k, g, w), rs in _by_signature(per_pass["busy"].get(label, [])).items():
                c = _median_counters(rs)
                gui = c.get("GRBM_GUI_ACTIVE", 0.0)
                cyc = gui / XCDS if gui else float("nan")
                mf = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * SIMDS) if gui else float("nan")
                busy_cu = c.get("SQ_BUSY_CU_CYCLES", 0.0)
                va = c.get("SQ_ACTIVE_INST_VALU", 0.0) / busy_cu if busy_cu else float("nan")
                la = c.get("SQ_ACTIVE_INST_LDS", 0.0) / busy_cu if busy_cu else float("nan")
                wt = c.get("SQ_WAIT_INST_ANY", 0.0) / max(1.0, c.get("SQ_WAVE_CYCLES", 0.0))
                bc = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(1.0, c.get("SQ_INSTS_LDS", 0.0))
                raw = " ".join(f"{n}={v:.0f}" for n, v in sorted(c.items()))
                lines.append(f"  {label:28s} {k[:44]:44s} {cyc:9.0f} {100 * mf:8.1f}% {100 * va:7.1f}% "
                             f"{100 * la:7.1f}% {100 * wt:5.1f}% {bc:7.2f}  {raw}")
                records.setdefault(label, {}).setdefault("activity", {})[f"{k} grid {g} wg {w}"] = {
                    "mfma_busy": round(mf, 4), "valu_active": round(va, 4), "lds_active": round(la, 4),
                    "wait": round(wt, 4), "bank_conflicts_per_lds_inst": round(bc, 3), "counters": c}
        lines.append("")

    cmd_path = os.path.join(d, "commands.txt")
    if os.path.exists(cmd_path):
        lines.append("Commands (run by python3 bench_profile.py --workload "
                     f"{workload} --out <dir>; <dir> here {out.replace(ROOT, '<repo>')}):")
        for line in open(cmd_path).read().splitlines():
            lines.append("  " + re.sub(r"\S*/(bench\.py|gpurun_out/)", r"<repo>/\1", line))
    return "\n".join(lines) + "\n", records


def _median_counters(rs: list[dict]) -> dict:
    if not rs:
        return {}
    names = set().union(*(r["counters"].keys() for r in rs))
    return {n: statistics.median(r["counters"].get(n, 0.0) for r in rs) for n in names}


def _read_bytes(c: dict) -> float:
    return 32 * c.get("TCC_EA0_RDREQ_32B", 0.0) + 64 * c.get("TCC_EA0_RDREQ_64B", 0.0) + 128 * c.get("TCC_EA0_RDREQ_128B", 0.0)


def _write_bytes(c: dict) -> float:
    w, w64 = c.get("TCC_EA0_WRREQ", 0.0), c.get("TCC_EA0_WRREQ_64B", 0.0)
    return 64 * w64 + 32 * (w - w64)


def write_profiles(workload: str, text: str, records: dict) -> None:
    sys.path.insert(0, ROOT)
    import bench
    name = PROFILE_NAMES.get(workload, workload)
    with open(os.path.join(PROFILES, f"{name}.txt"), "w") as fh:
        fh.write(text)
    path = os.path.join(PROFILES, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    for label, rec in records.items():
        if "bytes_per_launch" not in rec:
            continue
        data[label] = {"workload": workload, "alg_bytes": rec.get("alg_bytes"), "read_bytes": rec["read_bytes"],
                       "write_bytes": rec["write_bytes"], "bytes_per_launch": rec["bytes_per_launch"],
                       "calibration": rec.get("calibration"),
                       "method": "TCC_EA0 read/write requests by size (32/64/128 B)",
                       "kernel_source_hash": bench.kernel_source_hash(label)}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", action="append", required=True)
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--passes", default="bench,trace,reads,writes,busy")
    ap.add_argument("--parse-only", action="store_true", help="summarise results already under --out")
    ap.add_argument("--write", action="store_true", help="store the summary and traffic under profiles/")
    args = ap.parse_args()
    out = os.path.abspath(args.out)
    passes = args.passes.split(",")
    for w in args.workload:
        if not args.parse_only and not run_all(w, out, args.steps, passes):
            return 1
        text, records = summarize(w, out)
        with open(os.path.join(out, w, "summary.txt"), "w") as fh:
            fh.write(text)
        print(text, flush=True)
        if args.write:
            write_profiles(w, text, records)
    return 0


if __name__ == "__main__":
    sys.exit(main())
