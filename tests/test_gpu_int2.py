"""GPU parity of 2-bit rows (four codes per byte) against the CPU oracle:
range and greedy quantization and the baselines bit-exact, dequantize
bit-exact, the pooled lookup within 1e-5 * sum|terms| + 1e-6 with exact
error counts, the normalized l2 within 1e-12."""
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


DIMS = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
        257, 513, 1000, 1024]


@pytest.mark.parametrize("dim", DIMS)
def test_int2_range_and_greedy_bit_exact(q, dim):
    print("int2 quantize dim=%d" % dim, flush=True)
    g = np.random.default_rng(11000 + dim)
    x = special_rows(g, 600 + 7 if dim <= 256 else 150 + 3, dim)
    for mode in (oracle.RANGE, oracle.GREEDY):
        ref = oracle.quantize_rowwise(x, 2, mode, 200, 100)
        got = host(q.quantize_rowwise(dev(x), 2, mode, 200, 100))
        bad = np.nonzero(np.any(got != ref, axis=1))[0]
        assert bad.size == 0, (mode, bad[:8])
        y = host(q.dequantize(dev(ref), dim, 2))
        assert np.array_equal(y.view(np.uint32), oracle.dequantize(ref, dim, 2).view(np.uint32))


@pytest.mark.parametrize("method,param", [(oracle.SYMMETRIC, 0.0), (oracle.PERCENTILE, 0.95),
                                          (oracle.ACIQ, 0.0)])
@pytest.mark.parametrize("dim", [1, 3, 16, 33, 64, 128, 1000])
def test_int2_baselines_bit_exact(q, dim, method, param):
    g = np.random.default_rng(11100 + dim + 10 * method)
    x = special_rows(g, 500, dim)
    ref = oracle.quantize_baseline(x, 2, method, param)
    assert np.array_equal(host(q.quantize_baseline(dev(x), 2, method, param)), ref)


@pytest.mark.parametrize("dim", [1, 3, 16, 33, 64, 100, 128, 130, 256, 513, 1024])
@pytest.mark.parametrize("weighted", [False, True])
def test_int2_bag_ragged(q, dim, weighted):
    import torch
    g = np.random.default_rng(11200 + dim * 3 + weighted)
    rows = [1, 57, 300]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, 2)
    T, B = 3, 97
    lengths = g.integers(0, 71, size=T * B)
    lengths[::11] = 0
    offsets = np.concatenate([[0], np.cumsum(lengths)])
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lengths[gb]) for gb in range(T * B)])
    w = g.random(idx.size).astype(np.float32) if weighted else None
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = host(q.bag_forward(dev(packed), dev(toff), B, dim, 2, dev(idx.astype(np.int32)),
                             dev(offsets.astype(np.int32)), None if w is None else dev(w), err_count=err))
    ref, absd, rerr = oracle.bag_forward(packed, toff, B, dim, 2, idx.astype(np.int32),
                                         offsets.astype(np.int32), w)
    assert int(host(err)[0]) == rerr == 0
    assert_pooled_close(got, ref, absd, "int2 dim %d" % dim)
    empty = (lengths == 0).reshape(T, B).T
    assert np.all(got[empty] == 0) and not np.any(np.signbit(got[empty]))


@pytest.mark.parametrize("dim", [1, 16, 33, 64, 128, 200])
def test_int2_bag_short(q, dim):
    """Bags of 0..6 ids (fewer than 8 on average take the one-wave-per-bag
    kernel at every width), int64 ids, weighted."""
    import torch
    g = np.random.default_rng(11250 + dim)
    rows = [40, 3, 500]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, 2, oracle.GREEDY, 200, 100)
    T, B = 3, 211
    lengths = g.integers(0, 7, size=T * B)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lengths[gb]) for gb in range(T * B)])
    idx = idx.astype(np.int64)
    w = g.random(idx.size).astype(np.float32)
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = host(q.bag_forward(dev(packed), dev(toff), B, dim, 2, dev(idx), dev(offsets), dev(w),
                             err_count=err))
    ref, absd, rerr = oracle.bag_forward(packed, toff, B, dim, 2, idx, offsets, w)
    assert int(host(err)[0]) == rerr == 0
    assert_pooled_close(got, ref, absd, "int2 short dim %d" % dim)


@pytest.mark.parametrize("wid", [2, 3])
def test_int2_one_hot_ctr_shapes(q, wid):
    """The one-hot CTR workloads' shapes (one Zipf id per bag, sum pooling,
    int32 ids) over 2-bit rows, tables scaled down: several bags per wave."""
    w = synth.scaled(synth.workload(wid), rows=tuple(min(r, 5000) for r in synth.workload(wid).rows),
                     batch=300)
    x = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    packed = oracle.quantize_rowwise(x, 2)
    bt = synth.batch(w, index_dtype=np.int32)
    got = host(q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, w.dim, 2, dev(bt.indices),
                             dev(bt.offsets)))
    ref, absd, err = oracle.bag_forward(packed, bt.table_offsets, bt.B, w.dim, 2, bt.indices, bt.offsets)
    assert err == 0
    assert_pooled_close(got, ref, absd, "int2 one-hot workload %d" % wid)


def test_int2_bag_invalid_and_multi_hot(q):
    import torch
    g = np.random.default_rng(11300)
    dim, T, B = 64, 4, 50
    rows = [100, 10, 1, 40]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, 2)
    lengths = g.integers(0, 90, size=T * B)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = np.concatenate([g.integers(-5, rows[gb // B] + 5, size=lengths[gb])
                          for gb in range(T * B)]).astype(np.int64)
    offsets[17] = offsets[16] - 1
    offsets[90] = offsets[-1] + 3
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    wts = g.random(idx.size).astype(np.float32)
    for itype in (np.int32, np.int64):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = host(q.bag_forward(dev(packed), dev(toff), B, dim, 2, dev(idx.astype(itype)),
                                 dev(offsets.astype(itype)), dev(wts), err_count=err))
        ref, absd, rerr = oracle.bag_forward(packed, toff, B, dim, 2, idx.astype(itype),
                                             offsets.astype(itype), wts)
        assert int(host(err)[0]) == rerr and rerr > 20
        assert_pooled_close(got, ref, absd, "int2 invalid")
    # the multi-hot workload's shape, scaled
    w = synth.scaled(synth.workload(4), rows=(2000,) * 64, batch=200)
    xw = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    pw = oracle.quantize_rowwise(xw, 2)
    bt = synth.batch(w)
    got = host(q.bag_forward(dev(pw), dev(bt.table_offsets), bt.B, w.dim, 2, dev(bt.indices),
                             dev(bt.offsets), dev(bt.weights)))
    ref, absd, _ = oracle.bag_forward(pw, bt.table_offsets, bt.B, w.dim, 2, bt.indices, bt.offsets,
                                      bt.weights)
    assert_pooled_close(got, ref, absd, "int2 multi-hot")


def test_int2_l2(q):
    g = np.random.default_rng(11400)
    x = special_rows(g, 20000 + 3, 64)
    packed = oracle.quantize_rowwise(x, 2)
    ref = oracle.l2_error(x, packed, 2)
    got = q.l2_error(dev(x), dev(packed), 2)
    assert got["rows"] == ref["rows"]
    for k in ("mean_row", "sum_err2", "sum_x2"):
        assert abs(got[k] - ref[k]) <= 1e-12 * abs(ref[k]) + 1e-300, k
