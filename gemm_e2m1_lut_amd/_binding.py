"""ctypes binding of libe2m1lut.so (declared in include/e2m1lut.h).

Argument marshalling only: each function checks the torch tensors it is
given (device, dtype, shape, contiguity), allocates the output with torch when
none is passed, and calls the C entry point of the same name with raw device
pointers and the current HIP stream. Every step of the computation runs in the
library's kernels. A missing library raises at load time; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libe2m1lut.so")

ABI_VERSION = 2
DTYPE_F32 = 0
DTYPE_BF16 = 1
GEMV_MAX_BATCH = 16
TERNARY_MAX_BATCH = 16

_lib = None


class E2M1Error(RuntimeError):
    """A library call returned a negative status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the in-tree libe2m1lut.so (build it with `python -m gemm_e2m1_lut_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m gemm_e2m1_lut_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "e2m1_abi_version": (ctypes.c_int, []),
        "e2m1_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "dequant_decode": (ctypes.c_int, [vp, vp, vp, i64, i64, vp]),
        "dequant_gemv": (ctypes.c_int, [vp, vp, vp, vp, i32, i64, i64, i64, vp]),
        "dequant_gemm": (ctypes.c_int, [vp, vp, vp, vp, i32, i64, i64, i64, vp]),
        "dequant_gemv_grouped": (ctypes.c_int, [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                i32, vp]),
        "nm_spmm": (ctypes.c_int, [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp]),
        "mxfp4_quantize": (ctypes.c_int, [vp, vp, vp, i64, i64, vp]),
        "nvfp4_quantize": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp]),
        "ternary_gemv": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp]),
        "ternary_gemm_workspace_size": (sz, [i64, i64, i64]),
        "ternary_gemm": (ctypes.c_int, [vp, vp, vp, vp, vp, sz, i64, i64, i64, vp]),
        "ternary_wl_gemv": (ctypes.c_int, [ctypes.POINTER(vp), vp, vp, vp, vp, vp, i64, i64, vp]),
        "nvfp4_embedding_gather": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp]),
        "mxfp4_moe_workspace_size": (sz, [i64, i64, i64, i64, i64]),
        "mxfp4_moe_gemm": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64,
                                          i64, vp]),
        "mxfp4_moe_gemm_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                  vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    version = lib.e2m1_abi_version()
    if version != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {version}, binding expects {ABI_VERSION}")
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().e2m1_abi_version())


def strerror(status: int) -> str:
    return load_library().e2m1_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise E2M1Error(fn, status, strerror(status))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_U8 = (torch.uint8,)
_SCALE8 = (torch.uint8, torch.float8_e4m3fn)


# ----------------------------------------------------------------- decode --

def dequant_decode(packed: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """MXFP4 packed uint8 [rows, k/2] + E8M0 uint8 [rows, k/32] -> bf16 [rows, k]."""
    _need(packed, "packed", _U8)
    rows, half = packed.shape
    k = 2 * half
    _need(scales, "scales", _U8, (rows, k // 32))
    if out is None:
        out = torch.empty((rows, k), dtype=torch.bfloat16, device=packed.device)
    _need(out, "out", (torch.bfloat16, torch.int16), (rows, k))
    _check("dequant_decode", load_library().dequant_decode(_ptr(packed), _ptr(scales), _ptr(out),
                                                            rows, k, _stream(stream)))
    return out


# ------------------------------------------------------------------- GEMV --

def dequant_gemv(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor,
                 out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """y[b, n] = sum_k W[n, k] x[b, k]: W MXFP4 [n, k/2] + [n, k/32], x bf16 [batch, k] (or [k])."""
    _need(packed, "packed", _U8)
    n, half = packed.shape
    k = 2 * half
    _need(scales, "scales", _U8, (n, k // 32))
    squeeze = x.dim() == 1
    xb = x.unsqueeze(0) if squeeze else x
    _need(xb, "x", (torch.bfloat16,))
    batch = xb.shape[0]
    if xb.shape[1] != k:
        raise ValueError(f"x has {xb.shape[1]} columns, W has {k}")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if out is None:
        out = torch.empty((batch, n), dtype=out_dtype, device=packed.device)
    _need(out, "out", (out_dtype,), (batch, n))
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    _check("dequant_gemv", load_library().dequant_gemv(_ptr(packed), _ptr(scales), _ptr(xb), _ptr(out),
                                                        code, batch, n, k, _stream(stream)))
    return out[0] if squeeze else out


def dequant_gemv_grouped(mats, out_dtype: torch.dtype = torch.float32, outs=None, stream=None) -> list:
    """[y_g = W_g x_g for (packed_g, scales_g, x_g) in mats]: independent batch-1 products in shared launches.
    x_g is bf16 [k_g] (or [1, k_g]); y_g comes back with x_g's leading shape."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    mats = list(mats)
    if outs is not None and len(outs) != len(mats):
        raise ValueError(f"{len(outs)} outputs for {len(mats)} matrices")
    res, xs, ns, ks = [], [], [], []
    for g, (packed, scales, x) in enumerate(mats):
        _need(packed, "packed", _U8)
        n, half = packed.shape
        k = 2 * half
        _need(scales, "scales", _U8, (n, k // 32))
        squeeze = x.dim() == 1
        xb = x.unsqueeze(0) if squeeze else x
        _need(xb, "x", (torch.bfloat16,), (1, k))
        out = torch.empty((1, n), dtype=out_dtype, device=packed.device) if outs is None else outs[g]
        _need(out, "out", (out_dtype,), (1, n) if out.dim() == 2 else (n,))
        res.append(out[0] if (squeeze and out.dim() == 2) else out)
        xs.append(xb)
        ns.append(n)
        ks.append(k)
    cnt = len(mats)
    arr = ctypes.c_void_p * max(cnt, 1)
    a64 = ctypes.c_int64 * max(cnt, 1)
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    _check("dequant_gemv_grouped", load_library().dequant_gemv_grouped(
        cnt, arr(*[m[0].data_ptr() for m in mats]), arr(*[m[1].data_ptr() for m in mats]),
        arr(*[x.data_ptr() for x in xs]), arr(*[o.data_ptr() for o in res]), a64(*ns), a64(*ks), code,
        _stream(stream)))
    return res


def dequant_gemm(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
                 out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """MXFP4 W [n, k/2] + E8M0 [n, k/32], bf16 x [m, k] -> y [m, n] (fp32 accumulate), any m."""
    _need(packed, "packed", _U8)
    n, half = packed.shape
    k = 2 * half
    _need(scales, "scales", _U8, (n, k // 32))
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a [m, k] tensor")
    m = x.shape[0]
    _need(x, "x", (torch.bfloat16, torch.int16), (m, k))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=packed.device)
    _need(out, "out", (torch.float32, torch.bfloat16), (m, n))
    code = DTYPE_F32 if out.dtype == torch.float32 else DTYPE_BF16
    _check("dequant_gemm", load_library().dequant_gemm(_ptr(packed), _ptr(scales), _ptr(x), _ptr(out), code,
                                                        m, n, k, _stream(stream)))
    return out


def nm_spmm(values: torch.Tensor, meta: torch.Tensor, x: torch.Tensor, n_keep: int, m_group: int,
            out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """N:M sparse W (values bf16 [rows, (k/M) N], packed positions int32/uint32 [rows, words]) times
    bf16 x [batch, k] -> y [batch, rows]."""
    _need(values, "values", (torch.bfloat16, torch.int16))
    _need(meta, "meta", (torch.int32, torch.uint32))
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a [batch, k] tensor")
    batch, k = x.shape
    _need(x, "x", (torch.bfloat16, torch.int16))
    rows = values.shape[0]
    if m_group < 1 or k % m_group != 0 or values.shape[1] != (k // m_group) * n_keep:
        raise ValueError("values must hold (k / m_group) * n_keep entries per row")
    bits = 1 if m_group <= 2 else (m_group - 1).bit_length()
    words = -(-values.shape[1] // (32 // bits))
    _need(meta, "meta", (torch.int32, torch.uint32), (rows, words))
    if out is None:
        out = torch.empty((batch, rows), dtype=out_dtype, device=values.device)
    _need(out, "out", (torch.float32, torch.bfloat16), (batch, rows))
    code = DTYPE_F32 if out.dtype == torch.float32 else DTYPE_BF16
    _check("nm_spmm", load_library().nm_spmm(_ptr(values), _ptr(meta), _ptr(x), _ptr(out), code, batch, rows, k,
                                              n_keep, m_group, _stream(stream)))
    return out


# -------------------------------------------------------------- quantize --

def _bf16_rows(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a [rows, k] tensor")
    _need(x, name, (torch.bfloat16, torch.int16, torch.uint16))
    return x.shape


def mxfp4_quantize(x: torch.Tensor, out: tuple[torch.Tensor, torch.Tensor] | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 [rows, k] -> (codes uint8 [rows, k/2], E8M0 uint8 [rows, k/32])."""
    rows, k = _bf16_rows(x, "x")
    if out is None:
        out = (torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device),
               torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device))
    _need(out[0], "out[0]", _U8, (rows, k // 2))
    _need(out[1], "out[1]", _U8, (rows, k // 32))
    _check("mxfp4_quantize", load_library().mxfp4_quantize(_ptr(x), _ptr(out[0]), _ptr(out[1]), rows, k,
                                                            _stream(stream)))
    return out


def nvfp4_quantize(x: torch.Tensor, global_scale: torch.Tensor,
                   out: tuple[torch.Tensor, torch.Tensor] | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 [rows, k], fp32 global scale [1] -> (codes uint8 [rows, k/2], E4M3 bytes uint8 [rows, k/16])."""
    rows, k = _bf16_rows(x, "x")
    _need(global_scale, "global_scale", (torch.float32,))
    if global_scale.numel() != 1:
        raise ValueError("global_scale must hold one value")
    if out is None:
        out = (torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device),
               torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device))
    _need(out[0], "out[0]", _U8, (rows, k // 2))
    _need(out[1], "out[1]", _SCALE8, (rows, k // 16))
    _check("nvfp4_quantize", load_library().nvfp4_quantize(_ptr(x), _ptr(global_scale), _ptr(out[0]),
                                                            _ptr(out[1]), rows, k, _stream(stream)))
    return out


# ---------------------------------------------------------------- ternary --

def ternary_gemv(packed: torch.Tensor, row_scale: torch.Tensor, x: torch.Tensor,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Ternary W packed int32/uint32 [n, k/16] (16 weights per word), fp32 scale [n], fp32 x [k]."""
    _need(packed, "packed", (torch.int32, torch.uint32))
    n, words = packed.shape
    k = 16 * words
    _need(row_scale, "row_scale", (torch.float32,), (n,))
    _need(x, "x", (torch.float32,), (k,))
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _need(out, "out", (torch.float32,), (n,))
    _check("ternary_gemv", load_library().ternary_gemv(_ptr(packed), _ptr(row_scale), _ptr(x), _ptr(out),
                                                        n, k, _stream(stream)))
    return out


def ternary_gemm_workspace_size(batch: int, n: int, k: int) -> int:
    size = load_library().ternary_gemm_workspace_size(batch, n, k)
    if size == ctypes.c_size_t(-1).value:
        raise ValueError("invalid ternary GEMM extents")
    return int(size)


def ternary_gemm(packed: torch.Tensor, row_scale: torch.Tensor, x: torch.Tensor,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Ternary W packed int32/uint32 [n, k/16], fp32 scale [n], fp32 x [batch, k] -> y [batch, n].
    `workspace` (uint8, at least ternary_gemm_workspace_size bytes) is allocated when not given."""
    _need(packed, "packed", (torch.int32, torch.uint32))
    n, words = packed.shape
    k = 16 * words
    _need(row_scale, "row_scale", (torch.float32,), (n,))
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a [batch, k] tensor")
    batch = x.shape[0]
    _need(x, "x", (torch.float32,), (batch, k))
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=packed.device)
    _need(out, "out", (torch.float32,), (batch, n))
    need = ternary_gemm_workspace_size(batch, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=packed.device)
    if workspace is not None:
        _need(workspace, "workspace", _U8)
    _check("ternary_gemm", load_library().ternary_gemm(
        _ptr(packed), _ptr(row_scale), _ptr(x), _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel(), batch, n, k, _stream(stream)))
    return out


def ternary_wl_gemv(packed, scale: torch.Tensor, x_re: torch.Tensor, x_im: torch.Tensor,
                    out: tuple[torch.Tensor, torch.Tensor] | None = None,
                    stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Widely-linear complex ternary layer y = U x + W conj(x).

    packed: the four ternary matrices U_re, U_im, W_re, W_im, each int32/uint32
    [n, k/16] (a sequence of four tensors, or one [4, n, k/16] tensor);
    scale: fp32 [4, n] in the same order; x_re, x_im: fp32 [k].
    Returns (y_re, y_im), fp32 [n] each."""
    mats = list(packed.unbind(0)) if isinstance(packed, torch.Tensor) else list(packed)
    if len(mats) != 4:
        raise ValueError("packed must hold four matrices (U_re, U_im, W_re, W_im)")
    for i, m in enumerate(mats):
        _need(m, f"packed[{i}]", (torch.int32, torch.uint32))
    n, words = mats[0].shape
    for i, m in enumerate(mats):
        if tuple(m.shape) != (n, words):
            raise ValueError(f"packed[{i}] has shape {tuple(m.shape)}, expected {(n, words)}")
    k = 16 * words
    _need(scale, "scale", (torch.float32,), (4, n))
    _need(x_re, "x_re", (torch.float32,), (k,))
    _need(x_im, "x_im", (torch.float32,), (k,))
    if out is None:
        out = (torch.empty((n,), dtype=torch.float32, device=x_re.device),
               torch.empty((n,), dtype=torch.float32, device=x_re.device))
    _need(out[0], "out[0]", (torch.float32,), (n,))
    _need(out[1], "out[1]", (torch.float32,), (n,))
    ptrs = (ctypes.c_void_p * 4)(*[m.data_ptr() for m in mats])
    _check("ternary_wl_gemv", load_library().ternary_wl_gemv(ptrs, _ptr(scale), _ptr(x_re), _ptr(x_im),
                                                              _ptr(out[0]), _ptr(out[1]), n, k,
                                                              _stream(stream)))
    return out


# ----------------------------------------------------------------- gather --

def nvfp4_embedding_gather(table: torch.Tensor, block_scale: torch.Tensor, global_scale: torch.Tensor,
                           ids: torch.Tensor, out: torch.Tensor | None = None,
                           err_flag: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """NVFP4 table uint8 [vocab, hidden/2], E4M3 block scale [vocab, hidden/16], fp32 global
    scale [1] (device), int64 ids of any shape -> bf16 [*ids.shape, hidden]."""
    _need(table, "table", _U8)
    vocab, half = table.shape
    hidden = 2 * half
    _need(block_scale, "block_scale", _SCALE8, (vocab, hidden // 16))
    _need(global_scale, "global_scale", (torch.float32,), (1,))
    _need(ids, "ids", (torch.int64,))
    ntok = ids.numel()
    if out is None:
        out = torch.empty((*ids.shape, hidden), dtype=torch.bfloat16, device=table.device)
    _need(out, "out", (torch.bfloat16, torch.int16), (*ids.shape, hidden))
    if err_flag is not None:
        _need(err_flag, "err_flag", (torch.int32,), (1,))
    _check("nvfp4_embedding_gather",
           load_library().nvfp4_embedding_gather(_ptr(table), _ptr(block_scale), _ptr(global_scale),
                                                 _ptr(ids), _ptr(out), vocab, hidden, ntok,
                                                 _ptr(err_flag), _stream(stream)))
    return out


# -------------------------------------------------------------------- MoE --

def mxfp4_moe_workspace_size(tokens: int, hidden: int, inter: int, experts: int, topk: int) -> int:
    size = load_library().mxfp4_moe_workspace_size(tokens, hidden, inter, experts, topk)
    if size == ctypes.c_size_t(-1).value:
        raise ValueError("invalid MoE extents")
    return int(size)


def mxfp4_moe_gemm(x: torch.Tensor, w13: torch.Tensor, w13_scale: torch.Tensor, w2: torch.Tensor,
                   w2_scale: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """MXFP4 MoE layer: x bf16 [T, H]; w13 [E, 2I, H/2] + [E, 2I, H/32]; w2 [E, H, I/2] +
    [E, H, I/32]; topk_ids int32 [T, K]; topk_weights fp32 [T, K] -> bf16 [T, H]."""
    _need(x, "x", (torch.bfloat16,))
    tokens, hidden = x.shape
    _need(w13, "w13", _U8)
    experts, two_inter, _ = w13.shape
    inter = two_inter // 2
    _need(w13, "w13", _U8, (experts, 2 * inter, hidden // 2))
    _need(w13_scale, "w13_scale", _U8, (experts, 2 * inter, hidden // 32))
    _need(w2, "w2", _U8, (experts, hidden, inter // 2))
    _need(w2_scale, "w2_scale", _U8, (experts, hidden, inter // 32))
    _need(topk_ids, "topk_ids", (torch.int32,))
    topk = topk_ids.shape[1]
    _need(topk_ids, "topk_ids", (torch.int32,), (tokens, topk))
    _need(topk_weights, "topk_weights", (torch.float32,), (tokens, topk))
    if out is None:
        out = torch.empty((tokens, hidden), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", (torch.bfloat16,), (tokens, hidden))
    need = mxfp4_moe_workspace_size(tokens, hidden, inter, experts, topk)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", _U8)
    _check("mxfp4_moe_gemm",
           load_library().mxfp4_moe_gemm(_ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                         _ptr(topk_ids), _ptr(topk_weights), _ptr(out), _ptr(workspace),
                                         workspace.numel(), tokens, hidden, inter, experts, topk,
                                         _stream(stream)))
    return out


# Per-GPU workspace of mxfp4_moe_gemm_noalloc inside the library (E2M1_MOE_NOALLOC_WORKSPACE_BYTES).
MOE_NOALLOC_WORKSPACE_BYTES = 32 << 20


def mxfp4_moe_gemm_noalloc(x: torch.Tensor, w13: torch.Tensor, w13_scale: torch.Tensor, w2: torch.Tensor,
                           w2_scale: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                           out: torch.Tensor, stream=None) -> torch.Tensor:
    """mxfp4_moe_gemm with the library's own fixed per-GPU workspace: nothing is allocated,
    so `out` must be given. Calls that overlap on one GPU race (they share that workspace)."""
    _need(x, "x", (torch.bfloat16,))
    tokens, hidden = x.shape
    _need(w13, "w13", _U8)
    experts, two_inter, _ = w13.shape
    inter = two_inter // 2
    _need(w13, "w13", _U8, (experts, 2 * inter, hidden // 2))
    _need(w13_scale, "w13_scale", _U8, (experts, 2 * inter, hidden // 32))
    _need(w2, "w2", _U8, (experts, hidden, inter // 2))
    _need(w2_scale, "w2_scale", _U8, (experts, hidden, inter // 32))
    _need(topk_ids, "topk_ids", (torch.int32,))
    topk = topk_ids.shape[1]
    _need(topk_ids, "topk_ids", (torch.int32,), (tokens, topk))
    _need(topk_weights, "topk_weights", (torch.float32,), (tokens, topk))
    _need(out, "out", (torch.bfloat16,), (tokens, hidden))
    _check("mxfp4_moe_gemm_noalloc",
           load_library().mxfp4_moe_gemm_noalloc(_ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                                 _ptr(topk_ids), _ptr(topk_weights), _ptr(out), tokens, hidden,
                                                 inter, experts, topk, _stream(stream)))
    return out
