"""The C-ABI library loads, exports every entry point include/qemb.h
declares, and rejects bad arguments on the host before touching the GPU
(no compute call here)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle
from int4_row_wise_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    qbuild.ensure_built()
    from int4_row_wise_amd import qemb
    return qemb.load_library()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "qemb.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qemb_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(lib, s), s
    from int4_row_wise_amd import qemb
    assert sorted(qemb.EXPORTED) == syms


def test_abi_version_and_strerror(lib):
    assert lib.qemb_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -99):
        assert isinstance(lib.qemb_strerror(code), bytes)


def test_row_stride_matches_oracle(lib):
    for bits in (2, 4, 8):
        for dim in range(1, 1025):
            assert lib.qemb_row_stride(dim, bits) == oracle.row_stride(dim, bits)
    assert lib.qemb_row_stride(0, 4) == -1
    assert lib.qemb_row_stride(1025, 4) == -1
    assert lib.qemb_row_stride(16, 5) == -1 and lib.qemb_row_stride(16, 3) == -1


FAKE = ctypes.c_void_p(1 << 20)       # never dereferenced: validation fails first
MIS = ctypes.c_void_p((1 << 20) + 4)  # not 16-byte aligned


def test_quantize_argument_errors(lib):
    q = lib.qemb_quantize_rowwise
    assert q(FAKE, 10, 16, 5, 0, 200, 100, FAKE, None) == -1          # bits
    assert q(FAKE, 10, 0, 4, 0, 200, 100, FAKE, None) == -1           # dim
    assert q(FAKE, -1, 16, 4, 0, 200, 100, FAKE, None) == -1          # rows
    assert q(FAKE, 10, 16, 4, 2, 200, 100, FAKE, None) == -1          # clip mode
    assert q(FAKE, 10, 16, 4, 1, 100, 100, FAKE, None) == -1          # n_steps >= n_bins
    assert q(FAKE, 10, 16, 4, 1, 0, 0, FAKE, None) == -1              # n_bins < 1
    assert q(FAKE, 10, 1025, 4, 0, 200, 100, FAKE, None) == -3        # dim > max
    assert q(None, 10, 16, 4, 0, 200, 100, FAKE, None) == -1          # NULL x
    assert q(MIS, 10, 16, 4, 0, 200, 100, FAKE, None) == -2           # misaligned x
    assert q(FAKE, 10, 16, 4, 0, 200, 100, MIS, None) == -2           # misaligned out
    assert q(None, 0, 16, 4, 0, 200, 100, None, None) == 0            # nothing to do


def test_dequantize_argument_errors(lib):
    d = lib.qemb_dequantize
    assert d(FAKE, 10, 16, 3, FAKE, None) == -1
    assert d(None, 10, 16, 4, FAKE, None) == -1
    assert d(FAKE, 10, 16, 4, MIS, None) == -2
    assert d(FAKE, 10, 2000, 4, FAKE, None) == -3
    assert d(None, 0, 16, 4, None, None) == 0


def test_bag_argument_errors(lib):
    b = lib.qemb_bag_forward
    #          packed rows toff T  B  dim bits idx  offs nnz itype pool  w     out   err  stream
    assert b(FAKE, 10, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 2, 0, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 2, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 1, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, 4, None, FAKE, 5, 0, 0, None, FAKE, None, None) == -1
    assert b(FAKE, 10, None, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 0, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 0, None, MIS, None, None) == -2
    assert b(MIS, 10, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 0, None, FAKE, None, None) == -2
    assert b(FAKE, 10, FAKE, 2, 4, 4096, 4, FAKE, FAKE, 5, 0, 0, None, FAKE, None, None) == -3
    assert b(FAKE, -1, FAKE, 2, 4, 16, 4, FAKE, FAKE, 5, 0, 0, None, FAKE, None, None) == -1
    assert b(None, 0, None, 0, 4, 16, 4, None, None, 0, 0, 0, None, None, None, None) == 0
    assert b(None, 0, None, 3, 0, 16, 4, None, None, 0, 0, 0, None, None, None, None) == 0


def test_l2_argument_errors(lib):
    e = lib.qemb_l2_error
    assert lib.qemb_l2_error_workspace_bytes() > 0
    assert e(FAKE, FAKE, 10, 16, 4, None, FAKE, None) == -1
    assert e(FAKE, FAKE, 10, 16, 4, MIS, FAKE, None) == -2
    assert e(FAKE, FAKE, 10, 16, 7, FAKE, FAKE, None) == -1


def test_codebook_argument_errors(lib):
    for d in (1, 2, 15, 16, 17, 64, 128, 256, 1000, 1024):
        assert lib.qemb_codebook_row_stride(d) == oracle.codebook_row_stride(d)
    assert lib.qemb_codebook_row_stride(0) == -1 and lib.qemb_codebook_row_stride(1025) == -1
    qz = lib.qemb_quantize_codebook
    assert qz(FAKE, -1, 16, 10, FAKE, None) == -1
    assert qz(FAKE, 10, 0, 10, FAKE, None) == -1
    assert qz(FAKE, 10, 16, -1, FAKE, None) == -1
    assert qz(FAKE, 10, 2048, 10, FAKE, None) == -3
    assert qz(MIS, 10, 16, 10, FAKE, None) == -2
    assert qz(FAKE, 10, 16, 10, MIS, None) == -2
    assert qz(None, 10, 16, 10, FAKE, None) == -1
    assert qz(None, 0, 16, 10, None, None) == 0
    dq = lib.qemb_dequantize_codebook
    assert dq(FAKE, -1, 16, FAKE, None) == -1
    assert dq(FAKE, 10, 2048, FAKE, None) == -3
    assert dq(FAKE, 10, 16, MIS, None) == -2
    assert dq(None, 0, 16, None, None) == 0
    b = lib.qemb_bag_forward_codebook
    #          packed rows toff T  B  dim idx  offs nnz itype pool  w     out   err  stream
    assert b(FAKE, 10, FAKE, 2, 4, 16, FAKE, FAKE, 5, 2, 0, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, FAKE, FAKE, 5, 0, 2, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, FAKE, FAKE, 5, 0, 1, None, FAKE, None, None) == -1
    assert b(FAKE, 10, FAKE, 2, 4, 16, FAKE, FAKE, 5, 0, 0, None, MIS, None, None) == -2
    assert b(FAKE, 10, FAKE, 2, 4, 4096, FAKE, FAKE, 5, 0, 0, None, FAKE, None, None) == -3
    assert b(None, 0, None, 0, 4, 16, None, None, 0, 0, 0, None, None, None, None) == 0
    e = lib.qemb_l2_error_codebook
    assert e(FAKE, FAKE, 10, 16, None, FAKE, None) == -1
    assert e(FAKE, FAKE, 10, 16, MIS, FAKE, None) == -2
    assert e(FAKE, FAKE, 10, 2048, FAKE, FAKE, None) == -3


def test_interaction_argument_errors(lib):
    for T, d in ((0, 1), (1, 16), (26, 64), (64, 128), (1024, 1024)):
        assert lib.qemb_interaction_width(T, d) == oracle.interaction_width(T, d)
    assert lib.qemb_interaction_width(-1, 16) == -1 and lib.qemb_interaction_width(1025, 16) == -1
    assert lib.qemb_interaction_width(4, 0) == -1 and lib.qemb_interaction_width(4, 1025) == -1
    f = lib.qemb_dot_interaction
    #        dense pooled B  T  dim out   stream
    assert f(FAKE, FAKE, -1, 4, 16, FAKE, None) == -1
    assert f(FAKE, FAKE, 8, -1, 16, FAKE, None) == -1
    assert f(FAKE, FAKE, 8, 4, 0, FAKE, None) == -1
    assert f(FAKE, FAKE, 8, 4, 2048, FAKE, None) == -3
    assert f(FAKE, FAKE, 8, 2000, 16, FAKE, None) == -3
    assert f(None, FAKE, 8, 4, 16, FAKE, None) == -1
    assert f(FAKE, None, 8, 4, 16, FAKE, None) == -1
    assert f(FAKE, FAKE, 8, 4, 16, None, None) == -1
    assert f(MIS, FAKE, 8, 4, 16, FAKE, None) == -2
    assert f(FAKE, FAKE, 8, 4, 16, MIS, None) == -2
    assert f(None, None, 0, 4, 16, None, None) == 0


def test_binding_has_no_cpu_fallback(tmp_path):
    from int4_row_wise_amd import qemb
    saved = qemb._lib
    try:
        qemb._lib = None
        with pytest.raises(qemb.QembError):
            qemb.load_library(str(tmp_path / "missing.so"))
    finally:
        qemb._lib = saved


def test_baseline_argument_errors(lib):
    f = lib.qemb_quantize_baseline
    #        x     rows dim bits meth param packed stream
    assert f(FAKE, -1, 16, 4, 0, 0.0, FAKE, None) == -1
    assert f(FAKE, 10, 16, 5, 0, 0.0, FAKE, None) == -1
    assert f(FAKE, 10, 16, 3, 0, 0.0, FAKE, None) == -1
    assert f(FAKE, 10, 16, 4, 3, 0.0, FAKE, None) == -1
    assert f(FAKE, 10, 16, 4, 1, 0.4, FAKE, None) == -1
    assert f(FAKE, 10, 16, 4, 1, 1.5, FAKE, None) == -1
    assert f(FAKE, 10, 2048, 4, 0, 0.0, FAKE, None) == -3
    assert f(MIS, 10, 16, 4, 0, 0.0, FAKE, None) == -2
    assert f(FAKE, 10, 16, 4, 0, 0.0, MIS, None) == -2
    assert f(None, 0, 16, 4, 2, 0.0, None, None) == 0


def test_binding_checks_the_packed_row_width(lib):
    """The kernels index packed rows by the stride that dim and the row format
    imply; the binding rejects a tensor of another width or too few rows."""
    import torch
    from int4_row_wise_amd import qemb
    qemb._check_rows(torch.zeros((10, 80), dtype=torch.uint8), 80, 10)
    with pytest.raises(ValueError):
        qemb._check_rows(torch.zeros((10, 48), dtype=torch.uint8), 80, 10)
    with pytest.raises(ValueError):
        qemb._check_rows(torch.zeros((10, 80), dtype=torch.uint8), 80, 11)
    with pytest.raises(ValueError):
        qemb._check_rows(torch.zeros(800, dtype=torch.uint8), 80, 10)


def test_compress_sizes_and_argument_errors(lib):
    for d in (1, 7, 64, 128, 1000, 1024):
        for w in list(range(0, 33)):
            assert lib.qemb_compress_record_bytes(d, w) == oracle.record_bytes(d, w)
        assert lib.qemb_compress_bound(1000, d) == oracle.compress_bound(1000, d)
    assert lib.qemb_compress_record_bytes(0, 4) == -1 and lib.qemb_compress_record_bytes(16, 33) == -1
    assert lib.qemb_compress_record_bytes(1025, 4) == -1 and lib.qemb_compress_bound(-1, 16) == -1
    assert lib.qemb_compress_workspace_bytes(0) == 0
    assert lib.qemb_compress_workspace_bytes(1000) >= 8 * 16 + 1000
    mis4 = ctypes.c_void_p((1 << 20) + 2)   # not 4-byte aligned
    mis8 = ctypes.c_void_p((1 << 20) + 4)   # 4- but not 8-byte aligned
    f = lib.qemb_compress_pooled
    #        x     n    d   T  eb    out   offs  ws    stream
    assert f(FAKE, -1, 16, 1, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 0, 1, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 2048, 1, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert f(None, 10, 16, 1, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 16, 1, None, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 16, 1, FAKE, None, FAKE, FAKE, None) == -1
    assert f(FAKE, 10, 16, 1, FAKE, FAKE, None, FAKE, None) == -1
    assert f(FAKE, 10, 16, 1, FAKE, FAKE, FAKE, None, None) == -1
    assert f(MIS, 10, 16, 1, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, 10, 16, 1, FAKE, mis4, FAKE, FAKE, None) == -2
    assert f(FAKE, 10, 16, 1, FAKE, FAKE, mis8, FAKE, None) == -2
    assert f(FAKE, 10, 16, 1, FAKE, FAKE, FAKE, MIS, None) == -2
    g = lib.qemb_decompress_pooled
    #        in    bytes offs  n   d   T  eb    y     err   stream
    assert g(FAKE, 100, FAKE, -1, 16, 1, FAKE, FAKE, None, None) == -1
    assert g(FAKE, -1, FAKE, 10, 16, 1, FAKE, FAKE, None, None) == -1
    assert g(FAKE, 100, FAKE, 10, 16, 0, FAKE, FAKE, None, None) == -1
    assert g(FAKE, 100, FAKE, 10, 2048, 1, FAKE, FAKE, None, None) == -3
    assert g(FAKE, 100, None, 10, 16, 1, FAKE, FAKE, None, None) == -1
    assert g(FAKE, 100, FAKE, 10, 16, 1, None, FAKE, None, None) == -1
    assert g(FAKE, 100, FAKE, 10, 16, 1, FAKE, None, None, None) == -1
    assert g(None, 100, FAKE, 10, 16, 1, FAKE, FAKE, None, None) == -1
    assert g(mis4, 100, FAKE, 10, 16, 1, FAKE, FAKE, None, None) == -2
    assert g(FAKE, 100, mis8, 10, 16, 1, FAKE, FAKE, None, None) == -2
    assert g(FAKE, 100, FAKE, 10, 16, 1, FAKE, MIS, None, None) == -2
    assert g(None, 0, None, 0, 16, 1, None, None, None, None) == 0


def test_library_from_other_sources_is_refused(tmp_path, lib):
    """A library whose recorded source hash differs from the kernel sources
    now in the package (left from an older build) is refused before it is
    loaded; the current build is accepted."""
    import shutil

    from int4_row_wise_amd import qemb
    qemb.check_built_from_current_source(qbuild.LIB)
    stale = tmp_path / "libqemb.so"
    shutil.copy(qbuild.LIB, stale)
    with open(str(stale) + ".srchash", "w") as f:
        f.write("0" * 64 + "\n")
    with pytest.raises(qemb.QembError, match="other kernel sources"):
        qemb.check_built_from_current_source(str(stale))
    os.remove(str(stale) + ".srchash")
    with pytest.raises(qemb.QembError, match="other kernel sources"):
        qemb.check_built_from_current_source(str(stale))


def test_noalloc_compression_refuses_too_many_vectors_before_gpu_work(lib):
    """qemb_compress_pooled_noalloc checks n against its fixed workspace
    before any GPU call (the pointers are never touched here)."""
    from int4_row_wise_amd import qemb
    n = qemb.COMPRESS_NOALLOC_MAX_VECTORS + 1
    rc = lib.qemb_compress_pooled_noalloc(256, n, 32, 1, 256, 256, 256, None)
    assert rc == -5
    assert b"maximum" in lib.qemb_strerror(rc)
    assert lib.qemb_compress_pooled_noalloc(256, -1, 32, 1, 256, 256, 256, None) == -1
