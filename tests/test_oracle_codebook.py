"""Pins of the oracle's codebook quantization (16 fp32 levels per row from
1-D k-means, 4-bit codes): "Post-Training 4-bit Quantization on Embedding
Tables", review page, "Proposed method" (codebook quantization by k-means
clustering) and "Main findings" (lowest normalized l2 loss; 18.8%-37.5% of
the fp32 size).

Each check ties the oracle to something other than itself: the size range
the page prints, rows whose exact result is known in closed form, the
invariants of Lloyd iteration, an independently written numpy model (bit
for bit), the loss ordering the page reports, and torch's embedding_bag.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from tests import numpy_model as nm
from tests.gpu_common import special_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codebook_size_ratio.json")


def test_size_ratio_matches_the_printed_range():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        d = case["dim"]
        pct = 100.0 * oracle.codebook_row_stride(d) / (4 * d)
        assert round(pct, 1) == case["percent"], (d, pct)


def test_row_stride_layout():
    for d in (1, 2, 15, 16, 17, 64, 100, 256, 1024):
        S = oracle.codebook_row_stride(d)
        assert S % 16 == 0 and S >= 64 + (d + 1) // 2 and S - (64 + (d + 1) // 2) < 16


def _sse(x, y):
    return float(np.sum((x.astype(np.float64) - y.astype(np.float64)) ** 2, axis=-1).sum())


def test_grid_rows_are_reproduced_exactly():
    """A row made of the 16 grid levels (dyadic lo and step, so the grid is
    exact) is its own codebook: levels unchanged, zero error."""
    g = np.random.default_rng(1)
    for lo, step in ((-0.375, 0.0625), (0.5, 0.25), (-3.0, 0.125)):
        levels = np.float32(lo) + np.float32(step) * np.arange(16, dtype=np.float32)
        x = np.tile(levels, 4)
        g.shuffle(x)
        x = x[None, :].astype(np.float32)
        for it in (0, 1, 10):
            p = oracle.quantize_codebook(x, it)
            assert np.array_equal(oracle.codebook_levels(p)[0], levels)
            assert np.array_equal(oracle.dequantize_codebook(p, x.shape[1]), x)


def test_few_distinct_values_are_separated():
    """At most 16 distinct values, each pair farther apart than two grid
    steps, land in distinct clusters after one iteration: each value gets a
    code of its own and its level is the mean of equal values (exact up to
    the rounding of the fp32 sum and division: a few ulps)."""
    g = np.random.default_rng(2)
    for _ in range(50):
        m = int(g.integers(2, 17))
        gaps = g.uniform(2.2, 5.0, size=m - 1)
        vals = np.concatenate([[0.0], np.cumsum(gaps)])
        vals = vals / vals[-1] * g.uniform(0.01, 3.0) + g.uniform(-1, 1)
        vals = vals.astype(np.float32)
        if len(np.unique(vals)) < m:
            continue
        span = float(vals[-1] - vals[0])
        if np.min(np.diff(vals.astype(np.float64))) <= 2 * span / 15 * (1 + 1e-6):
            continue
        x = g.choice(vals, size=48)
        x[:m] = vals  # every value present
        x = x[None, :]
        p = oracle.quantize_codebook(x, 1)
        codes = oracle.codebook_codes(p, 48)[0]
        for v in vals:
            assert len(np.unique(codes[x[0] == v])) == 1
        assert len(np.unique(codes)) == m
        y = oracle.dequantize_codebook(p, 48)
        assert np.allclose(y, x, rtol=4 * 2.0 ** -23, atol=0)


def test_constant_row():
    x = np.full((1, 37), np.float32(-0.3), dtype=np.float32)
    p = oracle.quantize_codebook(x)
    assert np.all(oracle.codebook_levels(p) == np.float32(-0.3))
    assert np.all(oracle.codebook_codes(p, 37) == 0)
    assert np.array_equal(oracle.dequantize_codebook(p, 37), x)


def test_zero_iterations_is_the_uniform_grid():
    g = np.random.default_rng(3)
    x = (g.standard_normal((20, 64)) * 0.02).astype(np.float32)
    p = oracle.quantize_codebook(x, 0)
    for r in range(x.shape[0]):
        lo, hi = nm.row_range(x[r])
        delta = (np.float32(hi) - np.float32(lo)) / np.float32(15)
        grid = np.array([nm.fma32(np.float32(k), delta, lo) + np.float32(0.0) for k in range(16)],
                        dtype=np.float32)
        assert np.array_equal(oracle.codebook_levels(p)[r], grid)


def test_error_never_grows_with_iterations():
    """Lloyd iteration does not increase the squared error (up to the
    rounding of the fp32 means)."""
    g = np.random.default_rng(4)
    x = special_rows(g, 60, 64)
    x[np.abs(x) > 100] = 1.0
    prev = None
    for it in (0, 1, 2, 3, 5, 8, 13, 20):
        y = oracle.dequantize_codebook(oracle.quantize_codebook(x, it), 64)
        e = np.sum((x.astype(np.float64) - y) ** 2, axis=1)
        if prev is not None:
            assert np.all(e <= prev * (1 + 1e-5) + 1e-30)
        prev = e


def test_converged_rows_are_fixed_points():
    """After many iterations most rows no longer change: every code is the
    nearest level and every occupied level is the mean of its members."""
    g = np.random.default_rng(5)
    x = (g.standard_normal((100, 32)) * 0.02).astype(np.float32)
    a = oracle.quantize_codebook(x, 200)
    b = oracle.quantize_codebook(x, 201)
    same = np.all(a == b, axis=1)
    assert same.mean() >= 0.97
    lv, codes = oracle.codebook_levels(a), oracle.codebook_codes(a, 32)
    for r in np.nonzero(same)[0][:30]:
        dist = np.abs((x[r][:, None] - lv[r][None, :]).astype(np.float32))
        assert np.array_equal(codes[r], np.argmin(dist, axis=1))
        for k in range(16):
            m = codes[r] == k
            if m.any():
                mean = np.float32(nm.pairwise(np.where(m, x[r], np.float32(0))) / np.float32(m.sum()))
                assert lv[r][k] == mean + np.float32(0.0)


@pytest.mark.parametrize("dim", [1, 3, 16, 33, 64])
@pytest.mark.parametrize("n_iter", [0, 1, 10])
def test_oracle_matches_numpy_model(dim, n_iter):
    g = np.random.default_rng(600 + dim * 7 + n_iter)
    x = special_rows(g, 12, dim)
    x[np.abs(x) > 100] = 1.0
    p = oracle.quantize_codebook(x, n_iter)
    for r in range(x.shape[0]):
        assert np.array_equal(p[r], nm.encode_codebook(x[r], n_iter)), (r, x[r])


def test_loss_ordering_reported_by_the_page():
    """Mean normalized l2 at d=64 on N(0, 0.02) rows: codebook < greedy <
    range (the page reports the codebook loss lowest, the greedy lowest among
    uniform methods)."""
    g = np.random.default_rng(7)
    x = (g.standard_normal((300, 64)) * 0.02).astype(np.float32)
    cb = oracle.l2_error_codebook(x, oracle.quantize_codebook(x))["mean_row"]
    gr = oracle.l2_error(x, oracle.quantize_rowwise(x, 4, oracle.GREEDY, 200, 100), 4)["mean_row"]
    rg = oracle.l2_error(x, oracle.quantize_rowwise(x, 4), 4)["mean_row"]
    assert cb < gr < rg


def test_l2_codebook_matches_definition():
    g = np.random.default_rng(8)
    x = (g.standard_normal((40, 20)) * 0.05).astype(np.float32)
    p = oracle.quantize_codebook(x)
    y = oracle.dequantize_codebook(p, 20).astype(np.float64)
    xd = x.astype(np.float64)
    ratio = np.linalg.norm(xd - y, axis=1) / np.linalg.norm(xd, axis=1)
    got = oracle.l2_error_codebook(x, p)
    assert abs(got["mean_row"] - ratio.mean()) <= 1e-12
    assert abs(got["sum_err2"] - np.sum((xd - y) ** 2)) <= 1e-12 * np.sum((xd - y) ** 2)


def test_bag_codebook_matches_torch_embedding_bag():
    import torch
    g = np.random.default_rng(9)
    rows, dim, B = 50, 24, 16
    x = (g.standard_normal((rows, dim)) * 0.1).astype(np.float32)
    p = oracle.quantize_codebook(x)
    y = oracle.dequantize_codebook(p, dim).astype(np.float64)
    lengths = g.integers(0, 9, size=B)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = g.integers(0, rows, size=offs[-1]).astype(np.int64)
    w = g.random(idx.size).astype(np.float32)
    out, absd, err = oracle.bag_forward_codebook(p, np.array([0, rows], np.int64), B, dim, idx, offs, w)
    ref = torch.nn.functional.embedding_bag(torch.from_numpy(idx), torch.from_numpy(y),
                                            torch.from_numpy(offs[:-1]), mode="sum",
                                            per_sample_weights=torch.from_numpy(w.astype(np.float64)))
    assert err == 0
    assert np.allclose(out[:, 0, :], ref.numpy(), rtol=1e-12, atol=1e-15)
    # invalid ids are skipped and counted
    idx2 = idx.copy()
    idx2[::5] = rows + 3
    out2, _, err2 = oracle.bag_forward_codebook(p, np.array([0, rows], np.int64), B, dim, idx2, offs, w)
    assert err2 == int(np.sum(idx2 >= rows))
