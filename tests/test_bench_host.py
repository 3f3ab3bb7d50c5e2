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
