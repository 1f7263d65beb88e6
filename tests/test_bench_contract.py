"""Host-side checks of bench.py: the one-GPU refusal and the algorithmic byte
count behind its roofline fraction (no GPU needed).

The byte count follows the packed row layout of the row-wise quantizer
(Post-Training 4-bit Quantization on Embedding Tables, "Proposed method":
per row the codes plus an fp16 scale and an fp16 bias) and the pooled lookup
over CSR ids and offsets (DLRM review page, "Proposed method"): every lookup
reads one unpadded row, its id and its weight; every call reads the offsets
and writes one fp32 vector per bag.  Here that count is rebuilt from the
sizes of numpy arrays of those shapes, so a dropped or doubled term in
bench.py's formula fails."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration it does not run


def _bytes_from_arrays(nnz, n_bags, dim, bits, idx_dtype, weighted):
    codes = np.zeros(((dim * bits + 7) // 8,), np.uint8)      # one row's codes, unpadded
    params = np.zeros((2,), np.float16)                       # its scale and bias
    ids = np.zeros((nnz,), idx_dtype)
    weights = np.zeros((nnz if weighted else 0,), np.float32)
    offsets = np.zeros((n_bags + 1,), idx_dtype)
    out = np.zeros((n_bags, dim), np.float32)
    rows = nnz * (codes.nbytes + params.nbytes)
    return rows + ids.nbytes + weights.nbytes + offsets.nbytes + out.nbytes


@pytest.mark.parametrize("dim", [1, 3, 16, 64, 127, 128, 129, 512])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("idx_dtype", [np.int32, np.int64])
@pytest.mark.parametrize("weighted", [False, True])
def test_algorithmic_bag_bytes_match_array_sizes(dim, bits, idx_dtype, weighted):
    for nnz, n_bags in ((0, 1), (1, 1), (1000, 10), (4096, 7)):
        want = _bytes_from_arrays(nnz, n_bags, dim, bits, idx_dtype, weighted)
        got = bench.algorithmic_bag_bytes(nnz, n_bags, dim, bits, np.dtype(idx_dtype).itemsize,
                                          weighted)
        assert got == want, (nnz, n_bags, dim, bits, idx_dtype, weighted)


def test_headline_bytes_per_lookup():
    """INT4 rows of d = 128: 64 code bytes + 4 parameter bytes, an int32 id and
    an fp32 weight: 76 bytes per lookup, 512 output bytes and 4 offset bytes
    per bag (plus the closing offset)."""
    nnz, n_bags = 34075236, 64 * 16384
    got = bench.algorithmic_bag_bytes(nnz, n_bags, 128, 4, 4, True)
    assert got == nnz * 76 + (n_bags + 1) * 4 + n_bags * 512
    # the same call costs 3.13 GB at the workload's mean of 34.08 M lookups
    assert 3.12e9 < got < 3.14e9


@pytest.mark.parametrize("dim", [1, 2, 15, 16, 64, 128, 129])
@pytest.mark.parametrize("weighted", [False, True])
def test_algorithmic_codebook_bytes_match_array_sizes(dim, weighted):
    """Codebook rows (Post-Training 4-bit Quantization on Embedding Tables,
    "Proposed method", the k-means variant): 16 fp32 levels and one 4-bit
    code per element, unpadded."""
    for nnz, n_bags in ((0, 1), (5, 2), (1000, 10)):
        levels = np.zeros((16,), np.float32)
        codes = np.zeros(((dim + 1) // 2,), np.uint8)
        ids = np.zeros((nnz,), np.int32)
        weights = np.zeros((nnz if weighted else 0,), np.float32)
        offsets = np.zeros((n_bags + 1,), np.int32)
        out = np.zeros((n_bags, dim), np.float32)
        want = (nnz * (levels.nbytes + codes.nbytes) + ids.nbytes + weights.nbytes + offsets.nbytes
                + out.nbytes)
        assert bench.algorithmic_codebook_bytes(nnz, n_bags, dim, 4, weighted) == want
