"""Thin ctypes binding over libqemb.so (include/qemb.h).

Argument marshalling only: every step of quantization, decoding, pooling and
the error measurement runs in the HIP kernels behind the C ABI.  torch is
used for device memory (output allocation) and the current stream.  The
library is loaded on first use; if it was not built this raises -- there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqemb.so")

RANGE, GREEDY = 0, 1
SUM, WEIGHTED_SUM = 0, 1
INDEX_INT32, INDEX_INT64 = 0, 1
MAX_DIM = 1024

EXPORTED = (
    "qemb_abi_version", "qemb_strerror", "qemb_row_stride", "qemb_quantize_rowwise",
    "qemb_dequantize", "qemb_bag_forward", "qemb_l2_error_workspace_bytes", "qemb_l2_error",
    "qemb_codebook_row_stride", "qemb_quantize_codebook", "qemb_dequantize_codebook",
    "qemb_bag_forward_codebook", "qemb_l2_error_codebook", "qemb_interaction_width",
    "qemb_dot_interaction", "qemb_quantize_baseline", "qemb_compress_record_bytes",
    "qemb_compress_bound", "qemb_compress_workspace_bytes", "qemb_compress_pooled",
    "qemb_decompress_pooled", "qemb_compress_pooled_noalloc",
)

COMPRESS_VERBATIM = 32  # record header of a vector stored verbatim

SYMMETRIC, PERCENTILE, ACIQ = 0, 1, 2

CODEBOOK_ITERS = 10


class QembError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed: %s (%d)" % (fn, msg, code))
        self.code = code


_lib = None


def check_built_from_current_source(path: str = LIB_PATH) -> None:
    """Raise unless the library at `path` records (in `path`.srchash, written
    by the build) the hash of the kernel sources now in the package: a
    library left from older sources must not run in their place."""
    from int4_row_wise_amd import build as qbuild
    try:
        with open(path + ".srchash") as f:
            built = f.read().strip()
    except OSError:
        built = None
    now = qbuild.source_sha256()
    if built != now:
        raise QembError("load_library", -101,
                        "%s was built from other kernel sources (recorded %s, sources now %s); "
                        "rebuild with `python -m int4_row_wise_amd.build`" % (path, built, now))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QembError("load_library", -100,
                        "%s is not built (run `python -m int4_row_wise_amd.build`)" % path)
    check_built_from_current_source(path)
    L = ctypes.CDLL(path)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.qemb_abi_version.restype = ctypes.c_int
    L.qemb_strerror.argtypes = [ctypes.c_int]
    L.qemb_strerror.restype = ctypes.c_char_p
    L.qemb_row_stride.argtypes = [i32, i32]
    L.qemb_row_stride.restype = i64
    L.qemb_quantize_rowwise.argtypes = [p, i64, i32, i32, i32, i32, i32, p, p]
    L.qemb_quantize_rowwise.restype = ctypes.c_int
    L.qemb_dequantize.argtypes = [p, i64, i32, i32, p, p]
    L.qemb_dequantize.restype = ctypes.c_int
    L.qemb_bag_forward.argtypes = [p, i64, p, i32, i64, i32, i32, p, p, i64, i32, i32, p, p, p, p]
    L.qemb_bag_forward.restype = ctypes.c_int
    L.qemb_l2_error_workspace_bytes.restype = ctypes.c_size_t
    L.qemb_l2_error.argtypes = [p, p, i64, i32, i32, p, p, p]
    L.qemb_l2_error.restype = ctypes.c_int
    L.qemb_codebook_row_stride.argtypes = [i32]
    L.qemb_codebook_row_stride.restype = i64
    L.qemb_quantize_codebook.argtypes = [p, i64, i32, i32, p, p]
    L.qemb_quantize_codebook.restype = ctypes.c_int
    L.qemb_dequantize_codebook.argtypes = [p, i64, i32, p, p]
    L.qemb_dequantize_codebook.restype = ctypes.c_int
    L.qemb_bag_forward_codebook.argtypes = [p, i64, p, i32, i64, i32, p, p, i64, i32, i32, p, p, p, p]
    L.qemb_bag_forward_codebook.restype = ctypes.c_int
    L.qemb_l2_error_codebook.argtypes = [p, p, i64, i32, p, p, p]
    L.qemb_l2_error_codebook.restype = ctypes.c_int
    L.qemb_quantize_baseline.argtypes = [p, i64, i32, i32, i32, ctypes.c_float, p, p]
    L.qemb_quantize_baseline.restype = ctypes.c_int
    L.qemb_interaction_width.argtypes = [i32, i32]
    L.qemb_interaction_width.restype = i64
    L.qemb_dot_interaction.argtypes = [p, p, i64, i32, i32, p, p]
    L.qemb_dot_interaction.restype = ctypes.c_int
    L.qemb_compress_record_bytes.argtypes = [i32, i32]
    L.qemb_compress_record_bytes.restype = i64
    L.qemb_compress_bound.argtypes = [i64, i32]
    L.qemb_compress_bound.restype = i64
    L.qemb_compress_workspace_bytes.argtypes = [i64]
    L.qemb_compress_workspace_bytes.restype = ctypes.c_size_t
    L.qemb_compress_pooled.argtypes = [p, i64, i32, i32, p, p, p, p, p]
    L.qemb_compress_pooled.restype = ctypes.c_int
    L.qemb_decompress_pooled.argtypes = [p, i64, p, i64, i32, i32, p, p, p, p]
    L.qemb_decompress_pooled.restype = ctypes.c_int
    L.qemb_compress_pooled_noalloc.argtypes = [p, i64, i32, i32, p, p, p, p]
    L.qemb_compress_pooled_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise QembError(fn, rc, load_library().qemb_strerror(rc).decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(name: str, t: torch.Tensor, dtype=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def abi_version() -> int:
    return int(load_library().qemb_abi_version())


def row_stride(dim: int, bits: int) -> int:
    s = int(load_library().qemb_row_stride(dim, bits))
    if s < 0:
        raise ValueError("unsupported dim=%d bits=%d" % (dim, bits))
    return s


def _clip(mode) -> int:
    if isinstance(mode, str):
        return {"range": RANGE, "greedy": GREEDY}[mode]
    return int(mode)


def quantize_rowwise(x: torch.Tensor, bits: int = 4, clip_mode=RANGE, n_bins: int = 200,
                     n_steps: int = 100, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [rows, dim] float32 (device) -> packed [rows, stride] uint8."""
    _dev("x", x, torch.float32)
    rows, dim = x.shape
    S = row_stride(dim, bits)
    if out is None:
        out = torch.empty((rows, S), dtype=torch.uint8, device=x.device)
    _dev("out", out, torch.uint8)
    if tuple(out.shape) != (rows, S):
        raise ValueError("out must be [%d, %d]" % (rows, S))
    _check("qemb_quantize_rowwise", load_library().qemb_quantize_rowwise(
        _ptr(x), rows, dim, bits, _clip(clip_mode), n_bins, n_steps, _ptr(out), _stream(x)))
    return out


def quantize_baseline(x: torch.Tensor, bits: int = 4, method: int = SYMMETRIC, param: float = 0.0,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Baseline quantizers in the packed row format: SYMMETRIC, PERCENTILE
    (param = p in [0.5, 1]) or ACIQ.  x [rows, dim] float32 (device)."""
    _dev("x", x, torch.float32)
    rows, dim = x.shape
    S = row_stride(dim, bits)
    if out is None:
        out = torch.empty((rows, S), dtype=torch.uint8, device=x.device)
    _dev("out", out, torch.uint8)
    if tuple(out.shape) != (rows, S):
        raise ValueError("out must be [%d, %d]" % (rows, S))
    _check("qemb_quantize_baseline", load_library().qemb_quantize_baseline(
        _ptr(x), rows, dim, bits, int(method), float(param), _ptr(out), _stream(x)))
    return out


def dequantize(packed: torch.Tensor, dim: int, bits: int = 4,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """packed [rows, stride] uint8 (device) -> [rows, dim] float32."""
    _dev("packed", packed, torch.uint8)
    rows = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] != row_stride(dim, bits):
        raise ValueError("packed must be [rows, %d]" % row_stride(dim, bits))
    if out is None:
        out = torch.empty((rows, dim), dtype=torch.float32, device=packed.device)
    _dev("out", out, torch.float32)
    _check("qemb_dequantize", load_library().qemb_dequantize(
        _ptr(packed), rows, dim, bits, _ptr(out), _stream(packed)))
    return out


def _bag_args(packed, table_offsets, B, dim, indices, offsets, weights, pool_mode, out,
              err_count, total_rows):
    _dev("packed", packed, torch.uint8)
    _dev("table_offsets", table_offsets, torch.int64)
    _dev("indices", indices)
    _dev("offsets", offsets, indices.dtype)
    if indices.dtype == torch.int32:
        itype = INDEX_INT32
    elif indices.dtype == torch.int64:
        itype = INDEX_INT64
    else:
        raise TypeError("indices must be int32 or int64")
    T = table_offsets.numel() - 1
    if offsets.numel() != T * B + 1:
        raise ValueError("offsets must have T*B+1 = %d entries" % (T * B + 1))
    if pool_mode is None:
        pool_mode = SUM if weights is None else WEIGHTED_SUM
    if weights is not None:
        _dev("weights", weights, torch.float32)
        if weights.numel() != indices.numel():
            raise ValueError("weights must match indices")
    if out is None:
        out = torch.empty((B, T, dim), dtype=torch.float32, device=packed.device)
    _dev("out", out, torch.float32)
    if err_count is not None:
        _dev("err_count", err_count, torch.int32)
    if total_rows is None:
        total_rows = packed.shape[0]
    return T, itype, pool_mode, out, total_rows


def _check_rows(packed: torch.Tensor, stride: int, total_rows: int) -> None:
    """The packed tensor must hold total_rows rows of the expected stride:
    the kernels index it by that stride, so a mismatch would read past it."""
    if packed.dim() != 2 or packed.shape[1] != stride:
        raise ValueError("packed must be [rows, %d] for this dim and row format" % stride)
    if not 0 <= total_rows <= packed.shape[0]:
        raise ValueError("total_rows must be within the packed tensor's %d rows" % packed.shape[0])


def bag_forward(packed: torch.Tensor, table_offsets: torch.Tensor, B: int, dim: int, bits: int,
                indices: torch.Tensor, offsets: torch.Tensor, weights: Optional[torch.Tensor] = None,
                pool_mode: Optional[int] = None, out: Optional[torch.Tensor] = None,
                err_count: Optional[torch.Tensor] = None,
                total_rows: Optional[int] = None) -> torch.Tensor:
    """Pooled lookup: out [B, T, dim] float32; bag g = t*B + b spans
    indices[offsets[g]:offsets[g+1]] (ids local to table t)."""
    T, itype, pool_mode, out, total_rows = _bag_args(
        packed, table_offsets, B, dim, indices, offsets, weights, pool_mode, out, err_count,
        total_rows)
    _check_rows(packed, row_stride(dim, bits), total_rows)
    _check("qemb_bag_forward", load_library().qemb_bag_forward(
        _ptr(packed), total_rows, _ptr(table_offsets), T, B, dim, bits, _ptr(indices),
        _ptr(offsets), indices.numel(), itype, pool_mode, _ptr(weights), _ptr(out),
        _ptr(err_count), _stream(packed)))
    return out


def l2_error_workspace_bytes() -> int:
    return int(load_library().qemb_l2_error_workspace_bytes())


def l2_error(x: torch.Tensor, packed: torch.Tensor, bits: int,
             workspace: Optional[torch.Tensor] = None, out4: Optional[torch.Tensor] = None) -> dict:
    """Normalized l2 error of packed rows against x (binary64, on the device)."""
    _dev("x", x, torch.float32)
    _dev("packed", packed, torch.uint8)
    rows, dim = x.shape
    _check_rows(packed, row_stride(dim, bits), rows)
    if workspace is None:
        workspace = torch.empty(l2_error_workspace_bytes(), dtype=torch.uint8, device=x.device)
    if out4 is None:
        out4 = torch.empty(4, dtype=torch.float64, device=x.device)
    _check("qemb_l2_error", load_library().qemb_l2_error(
        _ptr(x), _ptr(packed), rows, dim, bits, _ptr(workspace), _ptr(out4), _stream(x)))
    return _l2_dict(out4)


def _l2_dict(out4: torch.Tensor) -> dict:
    v = out4.cpu().tolist()
    frob = (v[2] / v[3]) ** 0.5 if v[3] > 0 else 0.0
    return {"mean_row": v[0], "rows": int(v[1]), "sum_err2": v[2], "sum_x2": v[3], "frobenius": frob}


# ---- codebook rows (16 fp32 levels per row, 4-bit codes) ----

def codebook_row_stride(dim: int) -> int:
    s = int(load_library().qemb_codebook_row_stride(dim))
    if s < 0:
        raise ValueError("unsupported dim=%d" % dim)
    return s


def quantize_codebook(x: torch.Tensor, n_iter: int = CODEBOOK_ITERS,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [rows, dim] float32 (device) -> codebook rows [rows, stride] uint8."""
    _dev("x", x, torch.float32)
    rows, dim = x.shape
    S = codebook_row_stride(dim)
    if out is None:
        out = torch.empty((rows, S), dtype=torch.uint8, device=x.device)
    _dev("out", out, torch.uint8)
    if tuple(out.shape) != (rows, S):
        raise ValueError("out must be [%d, %d]" % (rows, S))
    _check("qemb_quantize_codebook", load_library().qemb_quantize_codebook(
        _ptr(x), rows, dim, n_iter, _ptr(out), _stream(x)))
    return out


def dequantize_codebook(packed: torch.Tensor, dim: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """codebook rows [rows, stride] uint8 (device) -> [rows, dim] float32."""
    _dev("packed", packed, torch.uint8)
    rows = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] != codebook_row_stride(dim):
        raise ValueError("packed must be [rows, %d]" % codebook_row_stride(dim))
    if out is None:
        out = torch.empty((rows, dim), dtype=torch.float32, device=packed.device)
    _dev("out", out, torch.float32)
    _check("qemb_dequantize_codebook", load_library().qemb_dequantize_codebook(
        _ptr(packed), rows, dim, _ptr(out), _stream(packed)))
    return out


def bag_forward_codebook(packed: torch.Tensor, table_offsets: torch.Tensor, B: int, dim: int,
                         indices: torch.Tensor, offsets: torch.Tensor,
                         weights: Optional[torch.Tensor] = None, pool_mode: Optional[int] = None,
                         out: Optional[torch.Tensor] = None,
                         err_count: Optional[torch.Tensor] = None,
                         total_rows: Optional[int] = None) -> torch.Tensor:
    """Pooled lookup over codebook rows; the same layout as bag_forward."""
    T, itype, pool_mode, out, total_rows = _bag_args(
        packed, table_offsets, B, dim, indices, offsets, weights, pool_mode, out, err_count,
        total_rows)
    _check_rows(packed, codebook_row_stride(dim), total_rows)
    _check("qemb_bag_forward_codebook", load_library().qemb_bag_forward_codebook(
        _ptr(packed), total_rows, _ptr(table_offsets), T, B, dim, _ptr(indices), _ptr(offsets),
        indices.numel(), itype, pool_mode, _ptr(weights), _ptr(out), _ptr(err_count),
        _stream(packed)))
    return out


def l2_error_codebook(x: torch.Tensor, packed: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None,
                      out4: Optional[torch.Tensor] = None) -> dict:
    """Normalized l2 error of codebook rows against x (binary64, on the device)."""
    _dev("x", x, torch.float32)
    _dev("packed", packed, torch.uint8)
    rows, dim = x.shape
    _check_rows(packed, codebook_row_stride(dim), rows)
    if workspace is None:
        workspace = torch.empty(l2_error_workspace_bytes(), dtype=torch.uint8, device=x.device)
    if out4 is None:
        out4 = torch.empty(4, dtype=torch.float64, device=x.device)
    _check("qemb_l2_error_codebook", load_library().qemb_l2_error_codebook(
        _ptr(x), _ptr(packed), rows, dim, _ptr(workspace), _ptr(out4), _stream(x)))
    return _l2_dict(out4)


# ---- dot interaction of the pooled embeddings ----

def interaction_width(T: int, dim: int) -> int:
    w = int(load_library().qemb_interaction_width(T, dim))
    if w < 0:
        raise ValueError("unsupported T=%d dim=%d" % (T, dim))
    return w


def dot_interaction(dense: torch.Tensor, pooled: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dense [B, d], pooled [B, T, d] float32 (device) -> [B, d + T(T+1)/2]:
    the dense vector, then the dot products of every pair of distinct rows of
    [dense; pooled] ((1,0), (2,0), (2,1), ...)."""
    _dev("dense", dense, torch.float32)
    _dev("pooled", pooled, torch.float32)
    if pooled.dim() != 3 or dense.dim() != 2:
        raise ValueError("dense must be [B, d] and pooled [B, T, d]")
    B, T, dim = pooled.shape
    if tuple(dense.shape) != (B, dim):
        raise ValueError("dense must be [%d, %d]" % (B, dim))
    W = interaction_width(T, dim)
    if out is None:
        out = torch.empty((B, W), dtype=torch.float32, device=dense.device)
    _dev("out", out, torch.float32)
    if tuple(out.shape) != (B, W):
        raise ValueError("out must be [%d, %d]" % (B, W))
    _check("qemb_dot_interaction", load_library().qemb_dot_interaction(
        _ptr(dense), _ptr(pooled), B, T, dim, _ptr(out), _stream(dense)))
    return out


# ---- error-bounded compression of pooled vectors (the all-to-all payload) ----

def compress_record_bytes(dim: int, w: int) -> int:
    r = int(load_library().qemb_compress_record_bytes(dim, w))
    if r < 0:
        raise ValueError("unsupported dim=%d w=%d" % (dim, w))
    return r


def compress_bound(n: int, dim: int) -> int:
    r = int(load_library().qemb_compress_bound(n, dim))
    if r < 0:
        raise ValueError("unsupported n=%d dim=%d" % (n, dim))
    return r


def compress_workspace_bytes(n: int) -> int:
    return int(load_library().qemb_compress_workspace_bytes(n))


def _vectors(x: torch.Tensor, T: Optional[int]):
    if x.dim() == 3:
        if T is not None and T != x.shape[1]:
            raise ValueError("T=%d does not match x of shape %s" % (T, tuple(x.shape)))
        return x.shape[0] * x.shape[1], x.shape[1], x.shape[2]
    if x.dim() != 2 or T is None:
        raise ValueError("x must be [B, T, d], or [n, d] with T given")
    return x.shape[0], T, x.shape[1]


def compress_pooled(x: torch.Tensor, eb: torch.Tensor, T: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, offs: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Error-bounded compression of pooled vectors x ([B, T, d], or [n, d]
    with T) under the per-table bounds eb ([T] float32, device).  Returns
    (out, offs): out is a uint8 buffer of compress_bound(n, d) bytes whose
    first offs[-1] bytes hold the records; offs is int64 [n + 1] on the
    device (reading offs[-1] on the host synchronizes)."""
    _dev("x", x, torch.float32)
    _dev("eb", eb, torch.float32)
    n, T, dim = _vectors(x, T)
    if eb.numel() != T:
        raise ValueError("eb must hold %d bounds" % T)
    if out is None:
        out = torch.empty(max(compress_bound(n, dim), 1), dtype=torch.uint8, device=x.device)
    if offs is None:
        offs = torch.empty(n + 1, dtype=torch.int64, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(compress_workspace_bytes(n), 16), dtype=torch.uint8, device=x.device)
    _dev("out", out, torch.uint8)
    _dev("offs", offs, torch.int64)
    _dev("workspace", workspace, torch.uint8)
    if out.numel() < compress_bound(n, dim) or offs.numel() != n + 1 or \
            workspace.numel() < compress_workspace_bytes(n):
        raise ValueError("out, offs or workspace too small")
    _check("qemb_compress_pooled", load_library().qemb_compress_pooled(
        _ptr(x), n, dim, T, _ptr(eb), _ptr(out), _ptr(offs), _ptr(workspace), _stream(x)))
    return out, offs


COMPRESS_NOALLOC_MAX_VECTORS = 1 << 21


def compress_pooled_noalloc(x: torch.Tensor, eb: torch.Tensor, out: torch.Tensor, offs: torch.Tensor,
                            T: Optional[int] = None):
    """compress_pooled for callers that cannot allocate: the library's
    workspace is a fixed per-GPU array (at most COMPRESS_NOALLOC_MAX_VECTORS
    vectors), and out (compress_bound(n, d) bytes) and offs ([n + 1] int64)
    are the caller's.  Calls that overlap on one GPU race on the array."""
    _dev("x", x, torch.float32)
    _dev("eb", eb, torch.float32)
    _dev("out", out, torch.uint8)
    _dev("offs", offs, torch.int64)
    n, T, dim = _vectors(x, T)
    if eb.numel() != T:
        raise ValueError("eb must hold %d bounds" % T)
    if out.numel() < compress_bound(n, dim) or offs.numel() != n + 1:
        raise ValueError("out or offs too small")
    _check("qemb_compress_pooled_noalloc", load_library().qemb_compress_pooled_noalloc(
        _ptr(x), n, dim, T, _ptr(eb), _ptr(out), _ptr(offs), _stream(x)))
    return out, offs


def decompress_pooled(buf: torch.Tensor, offs: torch.Tensor, dim: int, eb: torch.Tensor,
                      y: Optional[torch.Tensor] = None, err_count: Optional[torch.Tensor] = None,
                      in_bytes: Optional[int] = None) -> torch.Tensor:
    """Inverse of compress_pooled: records in buf (in_bytes of them, default
    the whole buffer) at offs ([n + 1] int64, device) -> y [n, d] float32.
    Malformed records decode as zeros and add 1 each to err_count."""
    _dev("buf", buf, torch.uint8)
    _dev("offs", offs, torch.int64)
    _dev("eb", eb, torch.float32)
    n = offs.numel() - 1
    if y is None:
        y = torch.empty((max(n, 0), dim), dtype=torch.float32, device=buf.device)
    _dev("y", y, torch.float32)
    if y.numel() != max(n, 0) * dim:
        raise ValueError("y must hold %d x %d values" % (n, dim))
    nb = buf.numel() if in_bytes is None else int(in_bytes)
    if nb > buf.numel():
        raise ValueError("in_bytes exceeds the buffer")
    _check("qemb_decompress_pooled", load_library().qemb_decompress_pooled(
        _ptr(buf), nb, _ptr(offs), n, dim, eb.numel(), _ptr(eb), _ptr(y), _ptr(err_count), _stream(buf)))
    return y
