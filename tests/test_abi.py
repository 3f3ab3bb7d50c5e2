"""CPU checks of the C ABI: the library loads, exports every function include/*.h
declares, and rejects bad arguments on the host before anything is launched.

No call here reaches a kernel launch: every argument set is rejected by
validation (or is an empty problem), so these run without a GPU.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

from conftest import ROOT

E2M1_OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_WS = 0, -1, -2, -3, -4, -5


def declared_functions() -> set[str]:
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    import gemm_e2m1_lut_amd as g
    return g.load_library()


def test_header_declares_the_five_operations():
    names = declared_functions()
    for op in ("dequant_decode", "dequant_gemv", "ternary_gemv", "ternary_gemm", "ternary_wl_gemv", "mxfp4_quantize", "nvfp4_quantize", "dequant_gemm", "nm_spmm", "nvfp4_embedding_gather",
               "mxfp4_moe_gemm", "mxfp4_moe_workspace_size", "ternary_gemm_workspace_size", "mxfp4_moe_gemm_noalloc", "e2m1_abi_version",
               "e2m1_strerror"):
        assert op in names


def test_library_exports_every_declared_function(lib):
    import gemm_e2m1_lut_amd as g
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = declared_functions() - exported
    assert not missing, missing
    for name in declared_functions():
        assert hasattr(lib, name)


def test_version_and_messages(lib):
    assert lib.e2m1_abi_version() == 2   # 2: ternary_gemm takes a workspace
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.e2m1_strerror(code)
    assert lib.e2m1_strerror(12345) == b"unknown status"


def P(addr: int) -> ctypes.c_void_p:
    """A fake device address: only ever seen by host-side validation here."""
    return ctypes.c_void_p(addr)


NULL = ctypes.c_void_p(0)
A, B, C, D = P(0x10000), P(0x20000), P(0x30000), P(0x40000)   # 16-byte aligned


def test_decode_validation(lib):
    f = lib.dequant_decode
    assert f(A, B, C, 4, 48, NULL) == E_SHAPE          # k % 32
    assert f(A, B, C, -1, 64, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, 0, 64, NULL) == E2M1_OK  # empty: nothing launched
    assert f(NULL, NULL, NULL, 5, 0, NULL) == E2M1_OK
    assert f(NULL, B, C, 4, 64, NULL) == E_NULL
    assert f(P(0x10008), B, C, 4, 64, NULL) == E_ALIGN
    assert f(A, B, P(0x30004), 4, 64, NULL) == E_ALIGN
    assert f(A, B, C, 2**62, 64, NULL) == E_SHAPE      # rows * k overflows


def test_gemv_validation(lib):
    f = lib.dequant_gemv
    assert f(A, B, C, D, 7, 1, 8, 64, NULL) == E_DTYPE
    assert f(A, B, C, D, 0, 0, 8, 64, NULL) == E_SHAPE   # batch 0
    assert f(A, B, C, D, 0, 17, 8, 64, NULL) == E_SHAPE  # batch above 16
    assert f(A, B, C, D, 0, 1, 8, 40, NULL) == E_SHAPE   # k % 32
    assert f(A, B, C, D, 0, 1, 2**31, 64, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, NULL, 0, 1, 0, 64, NULL) == E2M1_OK
    assert f(A, B, C, NULL, 0, 1, 8, 64, NULL) == E_NULL
    assert f(NULL, B, C, D, 1, 1, 8, 64, NULL) == E_NULL
    assert f(A, B, C, P(0x40002), 0, 1, 8, 64, NULL) == E_ALIGN   # fp32 y needs 4 bytes
    assert f(A, B, P(0x30008), D, 1, 1, 8, 64, NULL) == E_ALIGN   # x needs 16 bytes
    assert f(P(0x10001), B, C, D, 1, 1, 8, 64, NULL) == E_ALIGN


def test_gemv_grouped_validation(lib):
    f = lib.dequant_gemv_grouped
    vp, i64 = ctypes.c_void_p, ctypes.c_int64

    def call(count, packed, scales, x, y, n, k, dtype=0):
        arr = vp * max(len(packed), 1)
        a64 = i64 * max(len(n), 1)
        return f(count, arr(*packed), arr(*scales), arr(*x), arr(*y), a64(*n), a64(*k), dtype, NULL)

    ok = ([0x10000, 0x50000], [0x20000, 0x60000], [0x30000, 0x70000], [0x40000, 0x80000])
    assert call(2, *ok, [8, 8], [64, 64], dtype=7) == E_DTYPE
    assert call(65, *ok, [8, 8], [64, 64]) == E_SHAPE      # more matrices than the limit
    assert call(-1, *ok, [8, 8], [64, 64]) == E_SHAPE
    assert f(0, None, None, None, None, None, None, 0, NULL) == E2M1_OK
    assert f(1, None, None, None, None, None, None, 0, NULL) == E_NULL
    assert call(2, *ok, [8, 8], [64, 40]) == E_SHAPE       # k % 32 in the second matrix
    assert call(2, *ok, [8, 2**31], [64, 64]) == E_SHAPE
    assert call(2, ok[0], ok[1], ok[2], [0x40000, 0], [8, 8], [64, 64]) == E_NULL
    assert call(2, ok[0], ok[1], ok[2], [0, 0], [0, 0], [64, 64]) == E2M1_OK   # n = 0: nothing to write
    assert call(2, ok[0], [0x20000, 0], ok[2], ok[3], [8, 8], [64, 64]) == E_NULL
    assert call(2, ok[0], ok[1], ok[2], [0x40000, 0x80002], [8, 8], [64, 64]) == E_ALIGN   # fp32 y
    assert call(2, ok[0], ok[1], [0x30000, 0x70008], ok[3], [8, 8], [64, 64], 1) == E_ALIGN   # x
    assert call(2, [0x10000, 0x50001], ok[1], ok[2], ok[3], [8, 8], [64, 64], 1) == E_ALIGN


def test_ternary_validation(lib):
    f = lib.ternary_gemv
    assert f(A, B, C, D, 4, 24, NULL) == E_SHAPE   # k % 16
    assert f(A, B, C, D, -3, 16, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, NULL, 0, 16, NULL) == E2M1_OK
    assert f(A, B, C, NULL, 4, 16, NULL) == E_NULL
    assert f(NULL, B, C, D, 4, 16, NULL) == E_NULL
    assert f(P(0x10002), B, C, D, 4, 16, NULL) == E_ALIGN


def test_nm_validation(lib):
    f = lib.nm_spmm
    assert f(A, B, C, D, 5, 1, 8, 64, 2, 4, NULL) == E_DTYPE
    assert f(A, B, C, D, 0, 0, 8, 64, 2, 4, NULL) == E_SHAPE    # batch 0
    assert f(A, B, C, D, 0, 17, 8, 64, 2, 4, NULL) == E_SHAPE   # batch above 16
    assert f(A, B, C, D, 0, 1, 8, 64, 5, 4, NULL) == E_SHAPE    # n > m
    assert f(A, B, C, D, 0, 1, 8, 64, 2, 17, NULL) == E_SHAPE   # m > 16
    assert f(A, B, C, D, 0, 1, 8, 66, 2, 4, NULL) == E_SHAPE    # k % m
    assert f(NULL, NULL, NULL, NULL, 0, 1, 0, 64, 2, 4, NULL) == E2M1_OK
    assert f(A, NULL, C, D, 0, 1, 8, 64, 2, 4, NULL) == E_NULL
    assert f(A, P(0x20002), C, D, 0, 1, 8, 64, 2, 4, NULL) == E_ALIGN
    assert f(A, B, C, P(0x40002), 0, 1, 8, 64, 2, 4, NULL) == E_ALIGN


def test_gemm_validation(lib):
    f = lib.dequant_gemm
    assert f(A, B, C, D, 7, 4, 8, 64, NULL) == E_DTYPE
    assert f(A, B, C, D, 0, 4, 8, 40, NULL) == E_SHAPE     # k % 32
    assert f(A, B, C, D, 0, -1, 8, 64, NULL) == E_SHAPE
    assert f(A, B, C, D, 0, 2**31, 8, 64, NULL) == E_SHAPE
    assert f(A, B, C, D, 0, 4, 8, 8388576 + 32, NULL) == E_SHAPE   # k beyond the 32-bit tile offsets
    assert f(NULL, NULL, NULL, NULL, 0, 0, 8, 64, NULL) == E2M1_OK
    assert f(A, B, C, NULL, 0, 4, 8, 64, NULL) == E_NULL
    assert f(NULL, B, C, D, 1, 4, 8, 64, NULL) == E_NULL
    assert f(A, B, P(0x30008), D, 0, 4, 8, 64, NULL) == E_ALIGN
    assert f(A, B, C, P(0x40002), 0, 4, 8, 64, NULL) == E_ALIGN


def test_quantize_validation(lib):
    f = lib.mxfp4_quantize
    assert f(A, B, C, 4, 48, NULL) == E_SHAPE          # k % 32
    assert f(A, B, C, -1, 64, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, 0, 64, NULL) == E2M1_OK
    assert f(A, NULL, C, 4, 64, NULL) == E_NULL
    assert f(P(0x10008), B, C, 4, 64, NULL) == E_ALIGN   # x needs 16 bytes
    assert f(A, P(0x20004), C, 4, 64, NULL) == E_ALIGN   # codes need 8 bytes
    g = lib.nvfp4_quantize
    assert g(A, D, B, C, 4, 40, NULL) == E_SHAPE       # k % 16
    assert g(NULL, NULL, NULL, NULL, 3, 0, NULL) == E2M1_OK
    assert g(A, NULL, B, C, 4, 64, NULL) == E_NULL     # global scale
    assert g(A, P(0x40002), B, C, 4, 64, NULL) == E_ALIGN
    assert g(A, D, P(0x20001), C, 4, 64, NULL) == E_ALIGN


def test_ternary_gemm_validation(lib):
    f = lib.ternary_gemm
    W = P(0x70000)   # a 256-byte aligned workspace address
    assert f(A, B, C, D, W, 1 << 20, 0, 4, 16, NULL) == E_SHAPE    # batch 0
    assert f(A, B, C, D, W, 1 << 20, 17, 4, 16, NULL) == E_SHAPE   # batch above 16
    assert f(A, B, C, D, W, 1 << 20, 2, 4, 24, NULL) == E_SHAPE    # k % 16
    assert f(A, B, C, D, W, 1 << 20, 2, -1, 16, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, NULL, NULL, 0, 3, 0, 16, NULL) == E2M1_OK
    assert f(A, B, C, NULL, W, 1 << 20, 2, 4, 16, NULL) == E_NULL
    assert f(A, NULL, C, D, W, 1 << 20, 2, 4, 16, NULL) == E_NULL
    assert f(A, B, P(0x30002), D, W, 1 << 20, 2, 4, 16, NULL) == E_ALIGN
    assert f(P(0x10001), B, C, D, W, 1 << 20, 2, 4, 16, NULL) == E_ALIGN
    need = lib.ternary_gemm_workspace_size(8, 4, 64)
    assert f(A, B, C, D, NULL, 0, 8, 4, 64, NULL) == E_WS              # needed and missing
    assert f(A, B, C, D, W, need - 1, 8, 4, 64, NULL) == E_WS          # too small
    assert f(A, B, C, D, P(0x70010), need, 8, 4, 64, NULL) == E_ALIGN  # not 256-byte aligned


def test_ternary_gemm_workspace_size(lib):
    f = lib.ternary_gemm_workspace_size
    invalid = ctypes.c_size_t(-1).value
    assert f(1, 4, 4096) == 0 and f(4, 4, 4096) == 0   # batch 1 to 4: the one-launch kernels
    assert f(8, 4, 4096 + 16) == 0         # k % 64 != 0: ternary_gemv per row
    assert f(8, 0, 4096) == 0              # empty
    # per (group of two rows, 256-column slice): 4 KiB of digits and two exponents
    assert f(8, 4, 4096) == 4 * 16 * (4096 + 8)
    assert f(16, 4, 4096) == 8 * 16 * (4096 + 8)
    assert f(5, 4, 64 * 5) == 3 * 2 * (4096 + 8)
    assert f(0, 4, 64) == invalid and f(17, 4, 64) == invalid and f(2, 4, 24) == invalid


def test_ternary_wl_validation(lib):
    f = lib.ternary_wl_gemv
    mats = (ctypes.c_void_p * 4)(0x10000, 0x20000, 0x30000, 0x40000)
    E = P(0x50000)
    assert f(mats, A, B, C, D, E, 4, 24, NULL) == E_SHAPE    # k % 16
    assert f(mats, A, B, C, D, E, -1, 16, NULL) == E_SHAPE
    assert f(mats, A, B, C, D, E, 2**31, 16, NULL) == E_SHAPE
    assert f(None, NULL, NULL, NULL, NULL, NULL, 0, 16, NULL) == E2M1_OK   # empty
    assert f(mats, A, B, C, NULL, E, 4, 16, NULL) == E_NULL   # y_re
    assert f(mats, A, B, C, D, NULL, 4, 16, NULL) == E_NULL   # y_im
    assert f(None, A, B, C, D, E, 4, 16, NULL) == E_NULL      # no pointer array
    assert f(mats, NULL, B, C, D, E, 4, 16, NULL) == E_NULL   # scale
    gap = (ctypes.c_void_p * 4)(0x10000, 0x20000, 0, 0x40000)
    assert f(gap, A, B, C, D, E, 4, 16, NULL) == E_NULL
    odd = (ctypes.c_void_p * 4)(0x10000, 0x20002, 0x30000, 0x40000)
    assert f(odd, A, B, C, D, E, 4, 16, NULL) == E_ALIGN
    assert f(mats, A, B, P(0x30002), D, E, 4, 16, NULL) == E_ALIGN
    assert f(mats, A, B, C, D, P(0x50001), 4, 16, NULL) == E_ALIGN


def test_gather_validation(lib):
    f = lib.nvfp4_embedding_gather
    assert f(A, B, C, D, P(0x50000), 10, 24, 3, NULL, NULL) == E_SHAPE   # hidden % 16 (page guard)
    assert f(A, B, C, D, P(0x50000), -1, 32, 3, NULL, NULL) == E_SHAPE
    assert f(NULL, NULL, NULL, NULL, NULL, 10, 32, 0, NULL, NULL) == E2M1_OK
    assert f(A, B, NULL, D, P(0x50000), 10, 32, 3, NULL, NULL) == E_NULL
    assert f(NULL, B, C, D, P(0x50000), 10, 32, 3, NULL, NULL) == E_NULL
    assert f(A, B, C, D, P(0x50008), 10, 32, 3, NULL, NULL) == E_ALIGN   # out needs 16 bytes
    assert f(P(0x10004), B, C, D, P(0x50000), 10, 32, 3, NULL, NULL) == E_ALIGN


def test_moe_validation(lib):
    ws = lib.mxfp4_moe_workspace_size
    bad = ctypes.c_size_t(-1).value
    assert ws(4, 48, 64, 2, 1) == bad         # hidden % 32
    assert ws(4, 64, 40, 2, 1) == bad         # inter % 32
    assert ws(4, 64, 64, 0, 1) == bad         # no experts
    assert ws(4, 64, 64, 2, 0) == bad         # topk 0
    assert ws(0, 64, 64, 2, 1) == 0
    need = ws(256, 2880, 2880, 32, 4)
    assert 0 < need < 2**40
    f = lib.mxfp4_moe_gemm
    args = [A, B, C, D, P(0x50000), P(0x60000), P(0x70000), P(0x80000)]
    assert f(*args, P(0x90000), 0, 4, 64, 64, 2, 1, NULL) == E_WS
    small = ws(4, 64, 64, 2, 1)
    assert f(*args, P(0x90000), small - 1 if small else 0, 4, 64, 64, 2, 1, NULL) == E_WS
    assert f(*args, P(0x90010), small, 4, 64, 64, 2, 1, NULL) == E_ALIGN   # workspace 256-byte aligned
    assert f(*args, P(0x90000), small, 4, 48, 64, 2, 1, NULL) == E_SHAPE
    assert f(NULL, *args[1:], P(0x90000), small, 4, 64, 64, 2, 1, NULL) == E_NULL
    assert f(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 64, 64, 2, 1, NULL) == E2M1_OK


def test_moe_noalloc_validation(lib):
    """The no-allocation MoE rejects, on the host and before any GPU call, extents whose
    workspace exceeds its fixed per-GPU array."""
    f = lib.mxfp4_moe_gemm_noalloc
    ws = lib.mxfp4_moe_workspace_size
    limit = 32 << 20
    assert ws(485, 2880, 2880, 32, 4) <= limit < ws(486, 2880, 2880, 32, 4)
    args = [A, B, C, D, P(0x50000), P(0x60000), P(0x70000), P(0x80000)]
    assert f(*args, 486, 2880, 2880, 32, 4, NULL) == E_WS
    assert f(*args, 100000, 64, 64, 2, 1, NULL) == E_WS
    assert f(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 486, 2880, 2880, 32, 4, NULL) == E_WS
    assert f(*args, 4, 48, 64, 2, 1, NULL) == E_SHAPE      # hidden % 32
    assert f(*args, 4, 64, 64, 513, 1, NULL) == E_SHAPE    # too many experts
    assert f(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 64, 2, 1, NULL) == E2M1_OK


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    import gemm_e2m1_lut_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        b.load_library()
