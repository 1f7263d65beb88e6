"""GPU parity of the quantizer baselines ("Post-Training 4-bit Quantization
on Embedding Tables", review page, "Proposed method": symmetric
quantization, histogram-based clipping, ACIQ) against the CPU oracle:
packed rows bit-exact; the lookup and the l2 error read them unchanged."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from int4_row_wise_amd import synth
from tests.gpu_common import assert_pooled_close, dev, host, require_gpu, special_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    return require_gpu()


DIMS = [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 64, 65, 100, 127, 128, 129, 256, 257, 513, 1000, 1024]
METHODS = [(oracle.SYMMETRIC, 0.0), (oracle.PERCENTILE, 0.99), (oracle.ACIQ, 0.0)]


@pytest.mark.parametrize("method,param", METHODS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", DIMS)
def test_baseline_bit_exact(q, dim, bits, method, param):
    print("baseline method=%d bits=%d dim=%d" % (method, bits, dim), flush=True)
    g = np.random.default_rng(8000 + dim * 7 + bits + 100 * method)
    rows = 700 + 13 if dim <= 256 else 150 + 3
    x = special_rows(g, rows, dim)
    ref = oracle.quantize_baseline(x, bits, method, param)
    got = host(q.quantize_baseline(dev(x), bits, method, param))
    bad = np.nonzero(np.any(got != ref, axis=1))[0]
    assert bad.size == 0, "rows %s differ; first: x=%r gpu=%r oracle=%r" % (
        bad[:8], x[bad[0]][:8].tolist(), got[bad[0]][:24].tolist(), ref[bad[0]][:24].tolist())


@pytest.mark.parametrize("p", [0.5, 0.75, 0.9, 0.97, 0.999, 1.0])
@pytest.mark.parametrize("dim", [2, 7, 16, 64, 100, 1024])
def test_percentile_levels(q, dim, p):
    g = np.random.default_rng(8100 + dim)
    x = special_rows(g, 300, dim)
    for bits in (4, 8):
        ref = oracle.quantize_baseline(x, bits, oracle.PERCENTILE, p)
        assert np.array_equal(host(q.quantize_baseline(dev(x), bits, q.PERCENTILE, p)), ref), (bits, p)


def test_baselines_on_the_quantizer_workload_values(q):
    """200k rows of the quantizer workload (d = 64), every method, and the
    loss ordering the page reports on the GPU's own encodings."""
    w = synth.workload(5)
    x = synth.table_values_np(w, 0, 0, 200000)
    xd = dev(x)
    res = {}
    for method, param in METHODS:
        got = q.quantize_baseline(xd, 4, method, param)
        assert np.array_equal(host(got), oracle.quantize_baseline(x, 4, method, param)), method
        res[method] = q.l2_error(xd, got, 4)["mean_row"]
    rg = q.l2_error(xd, q.quantize_rowwise(xd, 4), 4)["mean_row"]
    assert rg <= min(res.values())


def test_lookup_reads_symmetric_rows(q):
    """The unchanged lookup over symmetric rows (bias -2^(b-1) s) matches the
    oracle's lookup of the oracle's rows."""
    w = synth.scaled(synth.workload(4), rows=(1500,) * 64, batch=100)
    x = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    bt = synth.batch(w)
    for bits in (4, 8):
        packed = oracle.quantize_baseline(x, bits, oracle.SYMMETRIC)
        got = host(q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, w.dim, bits, dev(bt.indices),
                                 dev(bt.offsets), dev(bt.weights)))
        ref, absd, _ = oracle.bag_forward(packed, bt.table_offsets, bt.B, w.dim, bits, bt.indices,
                                          bt.offsets, bt.weights)
        assert_pooled_close(got, ref, absd, "symmetric rows, %d bits" % bits)
        y = host(q.dequantize(dev(packed[:5000]), w.dim, bits))
        assert np.array_equal(y.view(np.uint32), oracle.dequantize(packed[:5000], w.dim, bits).view(np.uint32))
