"""Pins of the oracle's quantizer baselines ("Post-Training 4-bit
Quantization on Embedding Tables", review page, "Proposed method": the
comparison with ACIQ, histogram-based clipping and symmetric quantization;
"Main findings": the greedy search gives the lowest l2 loss among the
uniform methods, and earlier 4-bit methods do no better than range clipping
on small rows).

Each check ties the oracle to something other than itself: Lambert's W from
scipy for ACIQ's clip ratio, the Laplace error formula's first-order
condition, numpy's percentile, an independently written numpy model (bit for
bit), closed forms of the symmetric grid, and the loss ordering the page
reports.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from int4_row_wise_amd import synth
from tests import numpy_model as nm
from tests.gpu_common import special_rows


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_aciq_ratio_is_lambert_w(bits):
    from scipy.special import lambertw
    t = oracle.aciq_ratio(bits)
    assert abs(t - lambertw(3 * 4 ** bits).real) <= 1e-12 * t
    # first-order condition of 2 b^2 exp(-a/b) + a^2 / (3 4^M) at b = 1
    assert abs(-2 * np.exp(-t) + 2 * t / (3 * 4 ** bits)) < 1e-12


def _rows(seed, n, d):
    g = np.random.default_rng(seed)
    x = special_rows(g, n, d)
    x[np.abs(x) > 100] = 1.0
    return x


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dim", [1, 3, 16, 33, 64])
def test_baselines_match_numpy_model(dim, bits):
    x = _rows(700 + dim + bits, 12, dim)
    ratio = np.float32(oracle.aciq_ratio(bits))
    sym = oracle.quantize_baseline(x, bits, oracle.SYMMETRIC)
    pct = oracle.quantize_baseline(x, bits, oracle.PERCENTILE, 0.97)
    aq = oracle.quantize_baseline(x, bits, oracle.ACIQ)
    for r in range(x.shape[0]):
        assert np.array_equal(sym[r], nm.encode_symmetric(x[r], bits)), r
        lo, hi = nm.percentile_window(x[r], np.float32(0.97))
        assert np.array_equal(pct[r], nm.encode_window(x[r], bits, lo, hi)), r
        lo, hi = nm.aciq_window(x[r], bits, ratio)
        assert np.array_equal(aq[r], nm.encode_window(x[r], bits, lo, hi)), r


def test_percentile_window_is_numpy_percentile():
    g = np.random.default_rng(1)
    for d in (2, 5, 64, 100, 1000):
        for p in (0.5, 0.75, 0.9, 0.99, 0.999, 1.0):
            x = (g.standard_normal(d) * g.uniform(0.01, 10)).astype(np.float32)
            lo, hi = oracle.baseline_window(x, 4, oracle.PERCENTILE, p)
            ref = np.percentile(x.astype(np.float64), [100 * (1 - np.float64(np.float32(p))),
                                                      100 * np.float64(np.float32(p))])
            # h = (d - 1) p is rounded to binary32, which moves the
            # interpolation point by up to one ulp of d - 1
            tol = (4 * np.spacing(np.float32(np.max(np.abs(x)))) +
                   float(np.spacing(np.float32(d - 1))) * float(np.ptp(x)))
            assert abs(lo - ref[0]) <= tol and abs(hi - ref[1]) <= tol, (d, p, lo, hi, ref)


def test_percentile_one_is_range_quantization():
    x = _rows(2, 50, 64)
    for bits in (4, 8):
        assert np.array_equal(oracle.quantize_baseline(x, bits, oracle.PERCENTILE, 1.0),
                              oracle.quantize_rowwise(x, bits, oracle.RANGE))


def test_aciq_window_follows_the_laplace_scale():
    """On long Laplace rows the window is mean +- W(3 4^M) * mean|x - mean|
    (both estimated here in float64), kept inside the row range."""
    g = np.random.default_rng(3)
    x = g.laplace(0.1, 0.05, size=(20, 1024)).astype(np.float32)
    t = oracle.aciq_ratio(4)
    for r in range(20):
        lo, hi = oracle.baseline_window(x[r], 4, oracle.ACIQ)
        xd = x[r].astype(np.float64)
        mu = xd.mean()
        b = np.abs(xd - mu).mean()
        assert abs(lo - max(mu - t * b, xd.min())) <= 1e-5 * abs(b)
        assert abs(hi - min(mu + t * b, xd.max())) <= 1e-5 * abs(b)
        assert xd.min() <= lo <= hi <= xd.max()


def test_aciq_is_range_when_the_ratio_exceeds_the_range():
    """8-bit ACIQ clips at about 9.9 mean absolute deviations, beyond any
    point of a short Gaussian row, so it reproduces range quantization."""
    g = np.random.default_rng(4)
    x = (g.standard_normal((100, 16)) * 0.02).astype(np.float32)
    assert np.array_equal(oracle.quantize_baseline(x, 8, oracle.ACIQ), oracle.quantize_rowwise(x, 8))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_symmetric_grid_closed_forms(bits):
    H = 1 << (bits - 1)
    g = np.random.default_rng(5)
    # rows on the symmetric lattice s*q with s a power of two: exact round trip
    for k in range(-6, 3):
        s = np.float32(2.0 ** k)
        q = g.integers(-(H - 1), H, size=40)
        q[0] = H - 1  # max|x| = (H-1) s
        x = (q * s).astype(np.float32)[None]
        y = oracle.dequantize(oracle.quantize_baseline(x, bits, oracle.SYMMETRIC), 40, bits)
        assert np.array_equal(y, x)
    # zero stays zero and x -> -x mirrors the codes exactly
    x = _rows(6, 40, 33)
    x[:, 5] = 0.0
    p = oracle.quantize_baseline(x, bits, oracle.SYMMETRIC)
    pn = oracle.quantize_baseline(-x, bits, oracle.SYMMETRIC)
    y, yn = oracle.dequantize(p, 33, bits), oracle.dequantize(pn, 33, bits)
    assert np.all(y[:, 5] == 0)
    assert np.array_equal(yn, -y + 0.0)


def test_symmetric_scale_cap_keeps_the_bias_finite():
    x = np.array([[65504.0, -3.0, 1.0, 0.5]], np.float32)
    for bits in (2, 4, 8):
        y = oracle.dequantize(oracle.quantize_baseline(x, bits, oracle.SYMMETRIC), 4, bits)
        assert np.all(np.isfinite(y))
        H = 1 << (bits - 1)
        assert y[0, 0] == np.float32(65504.0 / H) * (H - 1)


def test_loss_ordering_reported_by_the_page():
    """On the quantizer workload's values (d = 64): codebook < greedy < range,
    and symmetric, 99th-percentile clipping and ACIQ do no better than
    range."""
    w = synth.workload(5)
    x = synth.table_values_np(w, 0, 0, 2000)

    def l2u(p):
        return oracle.l2_error(x, p, 4)["mean_row"]
    cb = oracle.l2_error_codebook(x, oracle.quantize_codebook(x))["mean_row"]
    gr = l2u(oracle.quantize_rowwise(x, 4, oracle.GREEDY, 200, 100))
    rg = l2u(oracle.quantize_rowwise(x, 4))
    others = [l2u(oracle.quantize_baseline(x, 4, oracle.SYMMETRIC)),
              l2u(oracle.quantize_baseline(x, 4, oracle.PERCENTILE, 0.99)),
              l2u(oracle.quantize_baseline(x, 4, oracle.ACIQ))]
    assert cb < gr < rg <= min(others)
