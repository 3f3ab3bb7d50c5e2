"""CPU oracle for the low-bit dequantisation hot path.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously-correct
reference the HIP library is checked against. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product package never does, and it imports nothing from the
product package. The arithmetic lives in ``oracle.c`` (plain C, fp64 unless a
page fixes the precision); this module marshals numpy arrays into it, builds
it with gcc when the shared object is missing, and adds one pure-Python
element loop for small cross-checks.

Pages followed (see the header of ``oracle.c`` for the section of each
function):
  * vLLM pull request 51583 digest (prhub.com.cn): MXFP4 unpack by bf16 lookup
    plus an integer add of the E8M0 scale into the exponent field, zero codes
    forced to +0.0.
  * SGLang pull request 34222 digest (prhub.com.cn): NVFP4 embedding,
    dequantised at gather time.
  * sglang-jax wiki page on the N:M structured sparse matmul: the Sparsifier's
    encode (top-N of a mask per group of M, positions bit-packed) and decode,
    and the sparse product.
  * FairyFuse blog post (blog.hotdry.top): 2-bit ternary GEMV with a per-row
    scale, and the widely-linear complex layer y = U x + W conj(x) over four
    such matrices.

Every function here is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, library routines (torch casts, numpy matmul)
and brute force on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, no intrinsics)."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _p(t):
    return ctypes.POINTER(t)


def load():
    """Load liboracle.so, building it first if it is missing or older than oracle.c."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, u8, u16, u32, f32, f64 = (ctypes.c_int64, ctypes.c_uint8, ctypes.c_uint16,
                                   ctypes.c_uint32, ctypes.c_float, ctypes.c_double)
    sig = {
        "or_abi_version": (ctypes.c_int, []),
        "or_threads": (ctypes.c_int, []),
        "or_set_threads": (None, [ctypes.c_int]),
        "or_e2m1_magnitude": (f64, [ctypes.c_int]),
        "or_bf16_from_double": (u16, [f64]),
        "or_double_from_bf16": (f64, [u16]),
        "or_bf16_from_double_array": (None, [_p(f64), _p(u16), i64]),
        "or_e4m3_to_double": (f64, [u8]),
        "or_mxfp4_decode_one": (u16, [ctypes.c_int, ctypes.c_int]),
        "or_mxfp4_decode": (ctypes.c_int, [_p(u8), _p(u8), _p(u16), i64, i64]),
        "or_mxfp4_gemv": (ctypes.c_int, [_p(u8), _p(u8), _p(u16), _p(f64), i64, i64, i64]),
        "or_ternary_gemv": (ctypes.c_int, [_p(u32), _p(f32), _p(f32), _p(f32), _p(f64), i64, i64]),
        "or_ternary_gemm": (ctypes.c_int, [_p(u32), _p(f32), _p(f32), _p(f32), _p(f64), i64, i64, i64]),
        "or_ternary_wl_gemv": (ctypes.c_int, [_p(_p(u32)), _p(f32), _p(f32), _p(f32), _p(f32), _p(f32),
                                              _p(f64), _p(f64), i64, i64]),
        "or_nvfp4_element": (u16, [ctypes.c_int, u8, f32]),
        "or_nvfp4_gather": (ctypes.c_int, [_p(u8), _p(u8), f32, _p(i64), _p(u16), i64, i64, i64,
                                           _p(i64)]),
        "or_e2m1_encode": (u8, [f64]),
        "or_e4m3_encode": (u8, [f64]),
        "or_mxfp4_quantize": (ctypes.c_int, [_p(u16), _p(u8), _p(u8), i64, i64]),
        "or_nvfp4_quantize": (ctypes.c_int, [_p(u16), f32, _p(u8), _p(u8), i64, i64]),
        "or_nm_bits": (ctypes.c_int, [ctypes.c_int]),
        "or_nm_encode": (ctypes.c_int, [_p(u16), _p(u8), _p(u16), _p(u32), i64, i64, ctypes.c_int, ctypes.c_int]),
        "or_nm_decode": (ctypes.c_int, [_p(u16), _p(u32), _p(u16), _p(u8), i64, i64, ctypes.c_int, ctypes.c_int]),
        "or_nm_spmm": (ctypes.c_int, [_p(u16), _p(u32), _p(u16), _p(f64), i64, i64, i64, ctypes.c_int,
                                      ctypes.c_int]),
        "or_mxfp4_moe": (ctypes.c_int, [_p(u16), _p(u8), _p(u8), _p(u8), _p(u8), _p(ctypes.c_int32),
                                        _p(f32), _p(f64), i64, i64, i64, i64, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(status, what):
    if status != 0:
        raise ValueError(f"oracle {what} rejected its input (status {status})")


def threads() -> int:
    return int(load().or_threads())


def set_threads(n: int) -> None:
    """Thread count of the OpenMP loops from now on (every result is independent of it)."""
    load().or_set_threads(int(n))


# ------------------------------------------------------------------ scalars --

def e2m1_magnitudes() -> list[float]:
    lib = load()
    return [lib.or_e2m1_magnitude(i) for i in range(8)]


def bf16_from_f64(values) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (single rounding, ties to even)."""
    v = _arr(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    load().or_bf16_from_double_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
    return out


def f64_from_bf16(bits) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(byte: int) -> float:
    return float(load().or_e4m3_to_double(int(byte) & 0xFF))


def mxfp4_decode_one(code: int, e8m0: int) -> int:
    return int(load().or_mxfp4_decode_one(int(code), int(e8m0)))


def nvfp4_element(code: int, block_scale_byte: int, global_scale) -> int:
    return int(load().or_nvfp4_element(int(code), int(block_scale_byte) & 0xFF,
                                       float(np.float32(global_scale))))


# ------------------------------------------------------------------- arrays --

def mxfp4_decode(packed, scales) -> np.ndarray:
    """packed uint8 [rows, k/2], scales uint8 [rows, k/32] -> bf16 bits [rows, k]."""
    p = _arr(packed, np.uint8)
    s = _arr(scales, np.uint8)
    rows, half = p.shape
    k = 2 * half
    assert s.shape == (rows, k // 32), (s.shape, rows, k)
    out = np.empty((rows, k), dtype=np.uint16)
    _check(load().or_mxfp4_decode(_ptr(p, ctypes.c_uint8), _ptr(s, ctypes.c_uint8),
                                  _ptr(out, ctypes.c_uint16), rows, k), "mxfp4_decode")
    return out


def mxfp4_gemv_f64(packed, scales, x_bits) -> np.ndarray:
    """y[b, n] = sum_k W[n, k] x[b, k] in fp64. x_bits: bf16 bits [batch, k]."""
    p = _arr(packed, np.uint8)
    s = _arr(scales, np.uint8)
    x = _arr(x_bits, np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    n, half = p.shape
    k = 2 * half
    batch = x.shape[0]
    assert x.shape == (batch, k) and s.shape == (n, k // 32)
    y = np.empty((batch, n), dtype=np.float64)
    _check(load().or_mxfp4_gemv(_ptr(p, ctypes.c_uint8), _ptr(s, ctypes.c_uint8),
                                _ptr(x, ctypes.c_uint16), _ptr(y, ctypes.c_double), batch, n, k),
           "mxfp4_gemv")
    return y


def mxfp4_gemv(packed, scales, x_bits, out_dtype: str = "f32") -> np.ndarray:
    """GEMV result rounded to the output type: 'f32' -> float32, 'bf16' -> bf16 bits."""
    y = mxfp4_gemv_f64(packed, scales, x_bits)
    if out_dtype == "f32":
        return y.astype(np.float32)
    if out_dtype == "bf16":
        return bf16_from_f64(y)
    if out_dtype == "f64":
        return y
    raise ValueError(out_dtype)


def ternary_gemv(packed, row_scale, x, want_f64: bool = False):
    """packed uint32 [n, k/16], row_scale f32 [n], x f32 [k] -> y f32 [n]."""
    p = _arr(packed, np.uint32)
    s = _arr(row_scale, np.float32)
    xv = _arr(x, np.float32)
    n, words = p.shape
    k = 16 * words
    assert s.shape == (n,) and xv.shape == (k,)
    y = np.empty(n, dtype=np.float32)
    y64 = np.empty(n, dtype=np.float64)
    _check(load().or_ternary_gemv(_ptr(p, ctypes.c_uint32), _ptr(s, ctypes.c_float),
                                  _ptr(xv, ctypes.c_float), _ptr(y, ctypes.c_float),
                                  _ptr(y64, ctypes.c_double), n, k), "ternary_gemv")
    return (y, y64) if want_f64 else y


def ternary_gemm(packed, row_scale, x, want_f64: bool = False):
    """packed uint32 [n, k/16], row_scale f32 [n], x f32 [batch, k] -> y f32 [batch, n]."""
    p = _arr(packed, np.uint32)
    s = _arr(row_scale, np.float32)
    xv = _arr(x, np.float32)
    n, words = p.shape
    k = 16 * words
    batch = xv.shape[0]
    assert s.shape == (n,) and xv.shape == (batch, k)
    y = np.empty((batch, n), dtype=np.float32)
    y64 = np.empty((batch, n), dtype=np.float64)
    _check(load().or_ternary_gemm(_ptr(p, ctypes.c_uint32), _ptr(s, ctypes.c_float),
                                  _ptr(xv, ctypes.c_float), _ptr(y, ctypes.c_float),
                                  _ptr(y64, ctypes.c_double), batch, n, k), "ternary_gemm")
    return (y, y64) if want_f64 else y


def ternary_wl_gemv(packed, scale, x_re, x_im, want_f64: bool = False):
    """Widely-linear complex ternary layer y = U x + W conj(x).

    packed: four uint32 [n, k/16] matrices (U_re, U_im, W_re, W_im), as a
    sequence or a [4, n, k/16] array; scale: f32 [4, n] in the same order;
    x_re, x_im: f32 [k]. Returns (y_re, y_im) as f32 [n], plus their fp64
    values when want_f64."""
    mats = [_arr(m, np.uint32) for m in packed]
    assert len(mats) == 4
    n, words = mats[0].shape
    k = 16 * words
    assert all(m.shape == (n, words) for m in mats)
    s = _arr(scale, np.float32)
    xr = _arr(x_re, np.float32)
    xi = _arr(x_im, np.float32)
    assert s.shape == (4, n) and xr.shape == (k,) and xi.shape == (k,)
    ptrs = (ctypes.POINTER(ctypes.c_uint32) * 4)(*[_ptr(m, ctypes.c_uint32) for m in mats])
    y = np.empty((2, n), dtype=np.float32)
    y64 = np.empty((2, n), dtype=np.float64)
    _check(load().or_ternary_wl_gemv(ptrs, _ptr(s, ctypes.c_float), _ptr(xr, ctypes.c_float),
                                     _ptr(xi, ctypes.c_float), _ptr(y[0], ctypes.c_float),
                                     _ptr(y[1], ctypes.c_float), _ptr(y64[0], ctypes.c_double),
                                     _ptr(y64[1], ctypes.c_double), n, k), "ternary_wl_gemv")
    return ((y[0], y[1]), (y64[0], y64[1])) if want_f64 else (y[0], y[1])


def e2m1_encode(v: float) -> int:
    return int(load().or_e2m1_encode(float(v)))


def e4m3_encode(t: float) -> int:
    return int(load().or_e4m3_encode(float(t)))


def mxfp4_quantize(x_bf16_bits):
    """bf16 bit patterns [rows, k] -> (codes uint8 [rows, k/2], E8M0 uint8 [rows, k/32])."""
    xv = _arr(x_bf16_bits, np.uint16)
    rows, k = xv.shape
    packed = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // 32), dtype=np.uint8)
    _check(load().or_mxfp4_quantize(_ptr(xv, ctypes.c_uint16), _ptr(packed, ctypes.c_uint8),
                                    _ptr(scales, ctypes.c_uint8), rows, k), "mxfp4_quantize")
    return packed, scales


def nvfp4_quantize(x_bf16_bits, global_scale: float):
    """bf16 bit patterns [rows, k], fp32 global scale -> (codes [rows, k/2], E4M3 bytes [rows, k/16])."""
    xv = _arr(x_bf16_bits, np.uint16)
    rows, k = xv.shape
    packed = np.empty((rows, k // 2), dtype=np.uint8)
    bs = np.empty((rows, k // 16), dtype=np.uint8)
    _check(load().or_nvfp4_quantize(_ptr(xv, ctypes.c_uint16), ctypes.c_float(float(np.float32(global_scale))),
                                    _ptr(packed, ctypes.c_uint8), _ptr(bs, ctypes.c_uint8), rows, k),
           "nvfp4_quantize")
    return packed, bs


def nm_layout(k: int, n: int, m: int):
    """(index bits, indices per word, kept values per row, words per row) of N:M sparsity."""
    bits = max(1, int(load().or_nm_bits(int(m))))
    packing = 32 // bits
    per_row = (k // m) * n
    return bits, packing, per_row, -(-per_row // packing)


def nm_encode(dense_bits, mask, n: int, m: int):
    """bf16 patterns [rows, k] + 0/1 mask -> (values bf16 [rows, (k/m) n], indices uint32 [rows, words])."""
    d = _arr(dense_bits, np.uint16)
    mk = _arr(mask, np.uint8)
    rows, k = d.shape
    _, _, per_row, words = nm_layout(k, n, m)
    vals = np.empty((rows, per_row), dtype=np.uint16)
    meta = np.empty((rows, words), dtype=np.uint32)
    _check(load().or_nm_encode(_ptr(d, ctypes.c_uint16), _ptr(mk, ctypes.c_uint8), _ptr(vals, ctypes.c_uint16),
                               _ptr(meta, ctypes.c_uint32), rows, k, n, m), "nm_encode")
    return vals, meta


def nm_decode(values, meta, k: int, n: int, m: int):
    """-> (dense bf16 patterns [rows, k], mask uint8 [rows, k])."""
    v = _arr(values, np.uint16)
    md = _arr(meta, np.uint32)
    rows = v.shape[0]
    dense = np.empty((rows, k), dtype=np.uint16)
    mask = np.empty((rows, k), dtype=np.uint8)
    _check(load().or_nm_decode(_ptr(v, ctypes.c_uint16), _ptr(md, ctypes.c_uint32), _ptr(dense, ctypes.c_uint16),
                               _ptr(mask, ctypes.c_uint8), rows, k, n, m), "nm_decode")
    return dense, mask


def nm_spmm(values, meta, x_bits, k: int, n: int, m: int) -> np.ndarray:
    """y [batch, rows] in fp64 = sparse W [rows, k] times bf16 x [batch, k]."""
    v = _arr(values, np.uint16)
    md = _arr(meta, np.uint32)
    x = _arr(x_bits, np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    rows, batch = v.shape[0], x.shape[0]
    y = np.empty((batch, rows), dtype=np.float64)
    _check(load().or_nm_spmm(_ptr(v, ctypes.c_uint16), _ptr(md, ctypes.c_uint32), _ptr(x, ctypes.c_uint16),
                             _ptr(y, ctypes.c_double), batch, rows, k, n, m), "nm_spmm")
    return y


def nvfp4_gather(table, block_scale, global_scale, ids):
    """Gather + dequantise rows -> (bf16 bits [ntok, hidden], count of bad ids)."""
    t = _arr(table, np.uint8)
    bs = _arr(block_scale, np.uint8)
    idv = _arr(ids, np.int64).reshape(-1)
    vocab, half = t.shape
    hidden = 2 * half
    assert bs.shape == (vocab, hidden // 16)
    out = np.empty((idv.size, hidden), dtype=np.uint16)
    bad = ctypes.c_int64(0)
    _check(load().or_nvfp4_gather(_ptr(t, ctypes.c_uint8), _ptr(bs, ctypes.c_uint8),
                                  float(np.float32(global_scale)), _ptr(idv, ctypes.c_int64),
                                  _ptr(out, ctypes.c_uint16), vocab, hidden, idv.size,
                                  ctypes.byref(bad)), "nvfp4_gather")
    return out, int(bad.value)


def nvfp4_gather_elementwise(table, block_scale, global_scale, ids) -> np.ndarray:
    """Pure-Python element loop in the order of the SGLang page's test reference.

    The page's reference multiplies in Python floats (fp64): value * (scale *
    global), and stores the product into a float32 tensor. Returns those
    float32 values [ntok, hidden]. Deliberately unvectorised; small inputs only.
    """
    mags = e2m1_magnitudes()
    ids = np.asarray(ids).reshape(-1)
    half = table.shape[1]
    hidden = 2 * half
    out = np.zeros((ids.size, hidden), dtype=np.float32)
    g = float(np.float32(global_scale))
    for t, rid in enumerate(ids):
        for c in range(hidden):
            byte = int(table[rid, c // 2])
            code = (byte & 0x0F) if c % 2 == 0 else (byte >> 4)
            magnitude = mags[code & 0x7]
            value = -magnitude if code & 0x8 else magnitude
            scale = e4m3_to_f64(block_scale[rid, c // 16]) * g
            out[t, c] = np.float32(value * scale)
    return out


def mxfp4_moe_f64(x_bits, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights) -> np.ndarray:
    """MXFP4 MoE layer in fp64 -> float64 [tokens, hidden] (before output rounding)."""
    x = _arr(x_bits, np.uint16)
    a13, s13 = _arr(w13, np.uint8), _arr(w13_scale, np.uint8)
    a2, s2 = _arr(w2, np.uint8), _arr(w2_scale, np.uint8)
    ids = _arr(topk_ids, np.int32)
    wts = _arr(topk_weights, np.float32)
    tokens, hidden = x.shape
    experts, two_inter, _ = a13.shape
    inter = two_inter // 2
    topk = ids.shape[1] if ids.ndim == 2 else 0
    assert a13.shape == (experts, 2 * inter, hidden // 2)
    assert s13.shape == (experts, 2 * inter, hidden // 32)
    assert a2.shape == (experts, hidden, inter // 2)
    assert s2.shape == (experts, hidden, inter // 32)
    assert ids.shape == (tokens, topk) and wts.shape == (tokens, topk)
    out = np.empty((tokens, hidden), dtype=np.float64)
    _check(load().or_mxfp4_moe(_ptr(x, ctypes.c_uint16), _ptr(a13, ctypes.c_uint8),
                               _ptr(s13, ctypes.c_uint8), _ptr(a2, ctypes.c_uint8),
                               _ptr(s2, ctypes.c_uint8), _ptr(ids, ctypes.c_int32),
                               _ptr(wts, ctypes.c_float), _ptr(out, ctypes.c_double),
                               tokens, hidden, inter, experts, topk), "mxfp4_moe")
    return out


def mxfp4_moe(x_bits, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights) -> np.ndarray:
    """MXFP4 MoE layer, output rounded once to bf16 bits [tokens, hidden]."""
    return bf16_from_f64(mxfp4_moe_f64(x_bits, w13, w13_scale, w2, w2_scale, topk_ids,
                                       topk_weights))
