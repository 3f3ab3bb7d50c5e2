"""Host-side pieces of bench.py (CPU): the source fingerprint that ties a committed
counter record in profiles/traffic.json to the kernel sources it was taken on."""
from __future__ import annotations

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402

SRC = '''// gemv -- header comment
#include "device.hpp"
/* a block
   comment */
__global__ void k(int* p) {   // trailing comment
    p[0] = 1;
}
'''


def test_comments_and_blank_space_do_not_change_the_code():
    edited = SRC.replace("header comment", "another header").replace("a block", "a longer block")
    edited = edited.replace("p[0] = 1;", "p[0]   =   1;") + "\n\n// added at the end\n"
    assert bench._code_only(SRC) == bench._code_only(edited)


def test_code_changes_do():
    assert bench._code_only(SRC) != bench._code_only(SRC.replace("p[0] = 1;", "p[0] = 2;"))
    assert bench._code_only(SRC) != bench._code_only(SRC.replace("int* p", "float* p"))


def test_every_committed_traffic_record_matches_its_sources():
    """A record whose kernels changed after its counters were taken is reported as null by
    bench.py; the committed ones are current."""
    import json
    with open(os.path.join(bench.PROFILES, "traffic.json")) as fh:
        records = json.load(fh)
    stale = [label for label, rec in records.items()
             if "kernel_source_hash" in rec and rec["kernel_source_hash"] != bench.kernel_source_hash(label)]
    assert stale == []


def test_build_flags_change_the_fingerprint():
    """A record taken under other compiler flags or another offload target is stale too."""
    flags = bench.build_fingerprint()
    assert "--offload-arch=" in flags
    same = bench.kernel_source_hash("gemv_b1_14336x4096", flags)
    assert same == bench.kernel_source_hash("gemv_b1_14336x4096")
    assert same != bench.kernel_source_hash("gemv_b1_14336x4096", flags.replace("xnack-", "xnack+"))
    assert same != bench.kernel_source_hash("gemv_b1_14336x4096", flags.replace("-O3", "-O2"))


def test_fingerprint_does_not_depend_on_where_the_tree_is():
    """The GPU runs use a copy of the tree at another path: the include paths in the flags must
    not change the hash."""
    from gemm_e2m1_lut_amd import build as hip_build
    moved = [f.replace(hip_build.ROOT, "/elsewhere/repo") for f in hip_build.HIPFLAGS]
    assert any(hip_build.ROOT in f for f in hip_build.HIPFLAGS)
    assert bench.build_fingerprint(moved, "/elsewhere/repo") == bench.build_fingerprint()
    assert "<repo>" in bench.build_fingerprint()


def test_cpu_description_names_the_host():
    d = bench.cpu_description()
    assert d.get("logical_processors", 0) >= 1
    assert d.get("affinity_cpus", 0) >= 1
    assert "model name" in d


def test_cpu_baseline_runs_the_oracle_on_one_core_too():
    import oracle

    class Fake(bench.Workload):
        def cpu_baseline(self, budget_s):
            return {"value": float(oracle.threads()), "unit": "GB/s", "cores": oracle.threads(),
                    "kind": "oracle", "sample": "fake"}

    n0 = oracle.threads()
    cpu = bench.run_cpu_baseline(Fake(), 0.0, 0.0)
    assert cpu["cores"] == n0 and cpu["single_core"]["cores"] == 1 and cpu["single_core"]["value"] == 1.0
    assert oracle.threads() == n0
    assert cpu["cpu"]["logical_processors"] >= 1


def test_profile_kernel_names():
    import bench_profile as bp
    assert bp.short_name("(anonymous namespace)::probe_empty_kernel<64>()") == "probe_empty_kernel<64>"
    assert bp.short_name("void e2m1::(anonymous namespace)::gemv_b1_rows_kernel<1, 2, 4, true>(e2m1::Args)") \
        == "gemv_b1_rows_kernel<1, 2, 4, true>"
    assert bp.short_name("void at::native::vectorized_elementwise_kernel<4, at::native::f(at::T&)::{lambda(float)#1}, "
                         "std::array<char*, 2ul> >(int, char*)").startswith("vectorized_elementwise_kernel<4,")


def test_every_workload_has_a_profile_name():
    """bench_profile.py names each workload's summary file; a workload added to bench.py
    without a name would write profiles/<workload>.txt under its bare key."""
    import bench
    import bench_profile as bp
    assert set(bench.WORKLOADS) == set(bp.PROFILE_NAMES)
    assert len(set(bp.PROFILE_NAMES.values())) == len(bp.PROFILE_NAMES)


def test_profile_records_are_attributed_by_marks():
    """Records between a label's mark and the next belong to that label, and so does every
    later record with the same kernel, grid and workgroup; the copies sit between two marks
    of MARK_BASE - 1."""
    import bench_profile as bp

    def rec(i, kernel, grid, wg=256):
        return {"id": i, "kernel": kernel, "grid": grid, "wg": wg, "counters": {}}

    def mark(i, g):
        return rec(i, "probe_empty_kernel<64>", g * 64, 64)

    recs = [mark(0, bp.MARK_BASE - 1), rec(1, "copy", 1 << 20), mark(2, bp.MARK_BASE - 1),
            rec(3, "fill", 512),
            mark(4, bp.MARK_BASE), rec(5, "k1", 1024), rec(6, "k2", 2048),
            mark(7, bp.MARK_BASE + 1), rec(8, "k1", 4096),
            mark(9, bp.MARK_BASE + 2),
            rec(10, "k1", 1024), rec(11, "k1", 4096), rec(12, "k2", 2048), rec(13, "fill", 512)]
    per, copies = bp.attribute(recs, ["a", "b"])
    assert [r["id"] for r in copies] == [1]
    assert [r["id"] for r in per["a"]] == [5, 6, 10, 12]
    assert [r["id"] for r in per["b"]] == [8, 11]
