"""CPU oracle for row-wise quantized embedding tables (test infrastructure).

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  It never touches the HIP library and the
HIP library never touches it: the two share no code.

The arithmetic lives in ``qemb_oracle.c`` (plain C, built with gcc, no
contraction, no fast-math).  This module only builds that file, loads it and
marshals numpy arrays.  What each function computes, and the passage of the
pages it follows, is stated in the C source:

* row-wise uniform quantization with fp16 scale and bias, range or greedy
  clipping ("Post-Training 4-bit Quantization on Embedding Tables", review
  page, "Proposed method" and "Main findings");
* two 4-bit codes per byte (DQRM repository page, Android demo paragraph);
* the pooled embedding-bag lookup ("Deep Learning Recommendation Model for
  Personalization and Recommendation Systems", review page, "Proposed
  method"), summed in binary64;
* the normalized l2 error (Post-Training 4-bit page, "Proposed method");
* codebook rows: 16 fp32 levels per row from 1-D k-means and 4-bit codes
  (Post-Training 4-bit page, "Proposed method" and "Main findings");
* error-bounded compression of the pooled embeddings devices exchange
  ("Avancées dans les recommandations en Deep Learning", scisimple page,
  "Méthodes de Compression des Données", "Stratégies de Compression
  Adaptative").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qemb_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = [
    "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
    "-fopenmp", "-shared", "-fPIC",
]

RANGE = 0
GREEDY = 1
SUM = 0
WEIGHTED_SUM = 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_row_stride.argtypes = [i32, i32]
        L.oracle_row_stride.restype = i64
        L.oracle_num_threads.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_f32_to_f16.argtypes = [p, p, i64]
        L.oracle_f16_to_f32.argtypes = [p, p, i64]
        L.oracle_quantize_rowwise.argtypes = [p, i64, i32, i32, i32, i32, i32, p, p]
        L.oracle_quantize_rowwise.restype = i32
        L.oracle_window_sse.argtypes = [p, i32, i32, i32, i32, i32]
        L.oracle_window_sse.restype = ctypes.c_float
        L.oracle_row_sse.argtypes = [p, p, i32, i32]
        L.oracle_row_sse.restype = ctypes.c_float
        L.oracle_dequantize.argtypes = [p, i64, i32, i32, p]
        L.oracle_dequantize.restype = i32
        L.oracle_bag_forward.argtypes = [p, i64, p, i32, i64, i32, i32, p, p, i64,
                                         i32, i32, p, p, p, p]
        L.oracle_bag_forward.restype = i32
        L.oracle_l2_error.argtypes = [p, p, i64, i32, i32, p]
        L.oracle_l2_error.restype = i32
        L.oracle_codebook_row_stride.argtypes = [i32]
        L.oracle_codebook_row_stride.restype = i64
        L.oracle_quantize_codebook.argtypes = [p, i64, i32, i32, p]
        L.oracle_quantize_codebook.restype = i32
        L.oracle_dequantize_codebook.argtypes = [p, i64, i32, p]
        L.oracle_dequantize_codebook.restype = i32
        L.oracle_bag_forward_codebook.argtypes = [p, i64, p, i32, i64, i32, p, p, i64,
                                                  i32, i32, p, p, p, p]
        L.oracle_bag_forward_codebook.restype = i32
        L.oracle_l2_error_codebook.argtypes = [p, p, i64, i32, p]
        L.oracle_l2_error_codebook.restype = i32
        L.oracle_aciq_ratio.argtypes = [i32]
        L.oracle_aciq_ratio.restype = ctypes.c_double
        L.oracle_baseline_window.argtypes = [p, i32, i32, i32, ctypes.c_float, p]
        L.oracle_baseline_window.restype = i32
        L.oracle_quantize_baseline.argtypes = [p, i64, i32, i32, i32, ctypes.c_float, p]
        L.oracle_quantize_baseline.restype = i32
        L.oracle_interaction_width.argtypes = [i32, i32]
        L.oracle_interaction_width.restype = i64
        L.oracle_dot_interaction.argtypes = [p, p, i64, i32, i32, p, p]
        L.oracle_dot_interaction.restype = i32
        L.oracle_record_bytes.argtypes = [i32, i32]
        L.oracle_record_bytes.restype = i64
        L.oracle_compress_bound.argtypes = [i64, i32]
        L.oracle_compress_bound.restype = i64
        L.oracle_compress_pooled.argtypes = [p, i64, i32, i32, p, p, p, p]
        L.oracle_compress_pooled.restype = i32
        L.oracle_decompress_pooled.argtypes = [p, i64, p, i64, i32, i32, p, p, p]
        L.oracle_decompress_pooled.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def row_stride(dim: int, bits: int) -> int:
    return int(lib().oracle_row_stride(dim, bits))


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_f16_to_f32(_ptr(h), _ptr(out), h.size)
    return out


def quantize_rowwise(x: np.ndarray, bits: int, clip_mode: int = RANGE,
                     n_bins: int = 200, n_steps: int = 100, return_window: bool = False):
    """Packed rows [rows, stride] (uint8); optionally the greedy (i, j) per row."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.shape
    S = row_stride(dim, bits)
    packed = np.zeros((rows, max(S, 0)), dtype=np.uint8)
    ij = np.zeros((rows, 2), dtype=np.int32)
    rc = lib().oracle_quantize_rowwise(_ptr(x), rows, dim, bits, clip_mode, n_bins, n_steps,
                                       _ptr(packed), _ptr(ij))
    if rc != 0:
        raise OracleError("oracle_quantize_rowwise returned %d" % rc)
    return (packed, ij) if return_window else packed


def window_sse(x_row: np.ndarray, bits: int, n_bins: int, i: int, j: int) -> np.float32:
    x_row = np.ascontiguousarray(x_row, dtype=np.float32)
    return np.float32(lib().oracle_window_sse(_ptr(x_row), x_row.size, bits, n_bins, i, j))


def row_sse(x_row: np.ndarray, packed_row: np.ndarray, bits: int) -> np.float32:
    x_row = np.ascontiguousarray(x_row, dtype=np.float32)
    packed_row = np.ascontiguousarray(packed_row, dtype=np.uint8)
    return np.float32(lib().oracle_row_sse(_ptr(x_row), _ptr(packed_row), x_row.size, bits))


def dequantize(packed: np.ndarray, dim: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    y = np.empty((rows, dim), dtype=np.float32)
    rc = lib().oracle_dequantize(_ptr(packed), rows, dim, bits, _ptr(y))
    if rc != 0:
        raise OracleError("oracle_dequantize returned %d" % rc)
    return y


def bag_forward(packed: np.ndarray, table_offsets: np.ndarray, B: int, dim: int, bits: int,
                indices: np.ndarray, offsets: np.ndarray, weights: np.ndarray | None = None,
                pool_mode: int | None = None, total_rows: int | None = None):
    """Returns (out[B, T, dim] float64, abs_terms[B, T, dim] float64, err_count)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    table_offsets = np.ascontiguousarray(table_offsets, dtype=np.int64)
    T = table_offsets.size - 1
    if indices.dtype == np.int32:
        itype = 0
    elif indices.dtype == np.int64:
        itype = 1
    else:
        raise TypeError("indices must be int32 or int64")
    indices = np.ascontiguousarray(indices)
    offsets = np.ascontiguousarray(offsets, dtype=indices.dtype)
    if pool_mode is None:
        pool_mode = SUM if weights is None else WEIGHTED_SUM
    if weights is not None:
        weights = np.ascontiguousarray(weights, dtype=np.float32)
    if total_rows is None:
        total_rows = packed.shape[0]
    out = np.empty((B, T, dim), dtype=np.float64)
    absd = np.empty((B, T, dim), dtype=np.float64)
    err = np.zeros(1, dtype=np.int64)
    rc = lib().oracle_bag_forward(_ptr(packed), total_rows, _ptr(table_offsets), T, B, dim, bits,
                                  _ptr(indices), _ptr(offsets), indices.size, itype, pool_mode,
                                  _ptr(weights), _ptr(out), _ptr(absd), _ptr(err))
    if rc != 0:
        raise OracleError("oracle_bag_forward returned %d" % rc)
    return out, absd, int(err[0])


def l2_error(x: np.ndarray, packed: np.ndarray, bits: int) -> dict:
    x = np.ascontiguousarray(x, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows, dim = x.shape
    out = np.zeros(4, dtype=np.float64)
    rc = lib().oracle_l2_error(_ptr(x), _ptr(packed), rows, dim, bits, _ptr(out))
    if rc != 0:
        raise OracleError("oracle_l2_error returned %d" % rc)
    frob = float(np.sqrt(out[2] / out[3])) if out[3] > 0 else 0.0
    return {"mean_row": float(out[0]), "rows": int(out[1]), "sum_err2": float(out[2]),
            "sum_x2": float(out[3]), "frobenius": frob}


# ---- codebook rows (16 fp32 levels per row from k-means, 4-bit codes) ----

CODEBOOK_ITERS = 10  # default Lloyd iterations


def codebook_row_stride(dim: int) -> int:
    return int(lib().oracle_codebook_row_stride(dim))


def quantize_codebook(x: np.ndarray, n_iter: int = CODEBOOK_ITERS) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.shape
    packed = np.empty((rows, codebook_row_stride(dim)), dtype=np.uint8)
    rc = lib().oracle_quantize_codebook(_ptr(x), rows, dim, n_iter, _ptr(packed))
    if rc != 0:
        raise OracleError("oracle_quantize_codebook returned %d" % rc)
    return packed


def codebook_levels(packed: np.ndarray) -> np.ndarray:
    """The 16 fp32 levels of each codebook row ([rows, 16])."""
    return np.ascontiguousarray(packed[:, :64]).view("<f4").reshape(-1, 16)


def codebook_codes(packed: np.ndarray, dim: int) -> np.ndarray:
    """The 4-bit codes of each codebook row ([rows, dim])."""
    b = packed[:, 64:64 + (dim + 1) // 2]
    codes = np.empty((packed.shape[0], 2 * b.shape[1]), dtype=np.uint8)
    codes[:, 0::2] = b & 15
    codes[:, 1::2] = b >> 4
    return codes[:, :dim]


def dequantize_codebook(packed: np.ndarray, dim: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    y = np.empty((rows, dim), dtype=np.float32)
    rc = lib().oracle_dequantize_codebook(_ptr(packed), rows, dim, _ptr(y))
    if rc != 0:
        raise OracleError("oracle_dequantize_codebook returned %d" % rc)
    return y


def bag_forward_codebook(packed: np.ndarray, table_offsets: np.ndarray, B: int, dim: int,
                         indices: np.ndarray, offsets: np.ndarray, weights: np.ndarray | None = None,
                         pool_mode: int | None = None, total_rows: int | None = None):
    """Returns (out[B, T, dim] float64, abs_terms[B, T, dim] float64, err_count)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    table_offsets = np.ascontiguousarray(table_offsets, dtype=np.int64)
    T = table_offsets.size - 1
    if indices.dtype == np.int32:
        itype = 0
    elif indices.dtype == np.int64:
        itype = 1
    else:
        raise TypeError("indices must be int32 or int64")
    indices = np.ascontiguousarray(indices)
    offsets = np.ascontiguousarray(offsets, dtype=indices.dtype)
    if pool_mode is None:
        pool_mode = SUM if weights is None else WEIGHTED_SUM
    if weights is not None:
        weights = np.ascontiguousarray(weights, dtype=np.float32)
    if total_rows is None:
        total_rows = packed.shape[0]
    out = np.empty((B, T, dim), dtype=np.float64)
    absd = np.empty((B, T, dim), dtype=np.float64)
    err = np.zeros(1, dtype=np.int64)
    rc = lib().oracle_bag_forward_codebook(_ptr(packed), total_rows, _ptr(table_offsets), T, B, dim,
                                           _ptr(indices), _ptr(offsets), indices.size, itype,
                                           pool_mode, _ptr(weights), _ptr(out), _ptr(absd),
                                           _ptr(err))
    if rc != 0:
        raise OracleError("oracle_bag_forward_codebook returned %d" % rc)
    return out, absd, int(err[0])


def l2_error_codebook(x: np.ndarray, packed: np.ndarray) -> dict:
    x = np.ascontiguousarray(x, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows, dim = x.shape
    out = np.zeros(4, dtype=np.float64)
    rc = lib().oracle_l2_error_codebook(_ptr(x), _ptr(packed), rows, dim, _ptr(out))
    if rc != 0:
        raise OracleError("oracle_l2_error_codebook returned %d" % rc)
    frob = float(np.sqrt(out[2] / out[3])) if out[3] > 0 else 0.0
    return {"mean_row": float(out[0]), "rows": int(out[1]), "sum_err2": float(out[2]),
            "sum_x2": float(out[3]), "frobenius": frob}


def interaction_width(T: int, dim: int) -> int:
    return int(lib().oracle_interaction_width(T, dim))


def dot_interaction(dense: np.ndarray, pooled: np.ndarray):
    """dense [B, d] float32, pooled [B, T, d] float32 -> (out [B, d + T(T+1)/2]
    float64, abs_terms of the same shape): the dense vector, then the dot
    products of every pair of distinct rows of Z = [dense; pooled], row by
    row (pairs (1,0), (2,0), (2,1), (3,0), ...)."""
    dense = np.ascontiguousarray(dense, dtype=np.float32)
    pooled = np.ascontiguousarray(pooled, dtype=np.float32)
    B, T, dim = pooled.shape
    if dense.shape != (B, dim):
        raise ValueError("dense must be [B, d]")
    W = interaction_width(T, dim)
    out = np.empty((B, W), dtype=np.float64)
    absd = np.empty((B, W), dtype=np.float64)
    rc = lib().oracle_dot_interaction(_ptr(dense), _ptr(pooled), B, T, dim, _ptr(out), _ptr(absd))
    if rc != 0:
        raise OracleError("oracle_dot_interaction returned %d" % rc)
    return out, absd


# ---- quantizer baselines (same packed rows as quantize_rowwise) ----

SYMMETRIC, PERCENTILE, ACIQ = 0, 1, 2


def aciq_ratio(bits: int) -> float:
    return float(lib().oracle_aciq_ratio(bits))


def baseline_window(x_row: np.ndarray, bits: int, method: int, param: float = 0.0):
    x_row = np.ascontiguousarray(x_row, dtype=np.float32)
    out = np.zeros(2, dtype=np.float32)
    rc = lib().oracle_baseline_window(_ptr(x_row), x_row.size, bits, method, param, _ptr(out))
    if rc != 0:
        raise OracleError("oracle_baseline_window returned %d" % rc)
    return out[0], out[1]


def quantize_baseline(x: np.ndarray, bits: int, method: int, param: float = 0.0) -> np.ndarray:
    """Packed rows (the quantize_rowwise format) by a baseline method:
    SYMMETRIC, PERCENTILE (param = p in [0.5, 1]) or ACIQ."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.shape
    S = row_stride(dim, bits)
    packed = np.zeros((rows, S), dtype=np.uint8)
    rc = lib().oracle_quantize_baseline(_ptr(x), rows, dim, bits, method, param, _ptr(packed))
    if rc != 0:
        raise OracleError("oracle_quantize_baseline returned %d" % rc)
    return packed


RAW_WIDTH = 32  # record header of a vector stored verbatim


def record_bytes(dim: int, w: int) -> int:
    return int(lib().oracle_record_bytes(dim, w))


def compress_bound(n: int, dim: int) -> int:
    return int(lib().oracle_compress_bound(n, dim))


def compress_pooled(x: np.ndarray, eb: np.ndarray):
    """x: [B][T][d] (or [n][d] with T = len(eb)) fp32 pooled vectors; eb: [T]
    per-table bounds.  Returns (buf uint8 [offs[-1]], offs int64 [n + 1],
    widths int32 [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    eb = np.ascontiguousarray(eb, dtype=np.float32).reshape(-1)
    T = eb.size
    dim = x.shape[-1]
    n = x.size // dim if dim else 0
    if x.ndim == 3:
        assert x.shape[1] == T, (x.shape, T)
    out = np.zeros(max(compress_bound(n, dim), 1), dtype=np.uint8)
    offs = np.zeros(n + 1, dtype=np.int64)
    widths = np.zeros(max(n, 1), dtype=np.int32)
    rc = lib().oracle_compress_pooled(_ptr(x), n, dim, T, _ptr(eb), _ptr(out), _ptr(offs), _ptr(widths))
    if rc != 0:
        raise OracleError("oracle_compress_pooled returned %d" % rc)
    return out[: offs[-1]].copy(), offs, widths[:n]


def decompress_pooled(buf: np.ndarray, offs: np.ndarray, dim: int, eb: np.ndarray):
    """Inverse of compress_pooled: returns (y fp32 [n][d], number of bad
    records)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    offs = np.ascontiguousarray(offs, dtype=np.int64)
    eb = np.ascontiguousarray(eb, dtype=np.float32).reshape(-1)
    n = offs.size - 1
    y = np.zeros((max(n, 0), dim), dtype=np.float32)
    bad = np.zeros(1, dtype=np.int64)
    rc = lib().oracle_decompress_pooled(_ptr(buf) if buf.size else None, buf.size, _ptr(offs), n, dim,
                                        eb.size, _ptr(eb), _ptr(y), _ptr(bad))
    if rc != 0:
        raise OracleError("oracle_decompress_pooled returned %d" % rc)
    return y, int(bad[0])
