"""GPU parity: every entry point of the HIP library against the CPU oracle on
the same seeded inputs, at oracle-sized shapes that span several tiles and
a ragged tail, plus the edge cases of the method.

Bars: packed rows (codes, fp16 scale/bias, padding) and dequantized values
bit-exact; error counts exact; pooled outputs within
|gpu - oracle| <= 1e-5 * sum_p |w_p * y_pj| + 1e-6 per element; the
normalized l2 error within 1e-12 relative (binary64 sums in another order).
"""
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


DIMS = [1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
        257, 511, 512, 513, 1000, 1024]


# ---------------------------------------------------------------------------
# quantizer: range
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", DIMS)
def test_range_quantize_bit_exact(q, dim, bits):
    print("range quantize dim=%d bits=%d" % (dim, bits), flush=True)
    g = np.random.default_rng(1000 * dim + bits)
    rows = 1000 + 37 if dim <= 256 else 300 + 5
    x = special_rows(g, rows, dim)
    ref = oracle.quantize_rowwise(x, bits, oracle.RANGE)
    got = host(q.quantize_rowwise(dev(x), bits, q.RANGE))
    assert np.array_equal(got, ref)
    y = host(q.dequantize(dev(ref), dim, bits))
    assert np.array_equal(y.view(np.uint32), oracle.dequantize(ref, dim, bits).view(np.uint32))


# ---------------------------------------------------------------------------
# quantizer: greedy
# ---------------------------------------------------------------------------

GREEDY_DIMS = [1, 2, 3, 7, 16, 20, 33, 64, 65, 100, 128, 200, 256, 300, 512, 1000, 1024]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", GREEDY_DIMS)
def test_greedy_quantize_bit_exact(q, dim, bits):
    print("greedy quantize dim=%d bits=%d" % (dim, bits), flush=True)
    g = np.random.default_rng(2000 * dim + bits)
    rows = 700 + 13 if dim <= 128 else 130 + 3
    x = special_rows(g, rows, dim)
    ref = oracle.quantize_rowwise(x, bits, oracle.GREEDY, 200, 100)
    got = host(q.quantize_rowwise(dev(x), bits, q.GREEDY, 200, 100))
    mism = np.nonzero((got != ref).any(axis=1))[0]
    assert mism.size == 0, "rows differ: %s" % mism[:10]


@pytest.mark.parametrize("n_bins,n_steps", [(1, 0), (2, 1), (7, 3), (16, 15), (200, 0), (50, 49)])
@pytest.mark.parametrize("dim", [3, 16, 64, 100])
def test_greedy_search_parameters(q, dim, n_bins, n_steps):
    g = np.random.default_rng(7 * dim + n_bins)
    x = special_rows(g, 300, dim)
    ref = oracle.quantize_rowwise(x, 4, oracle.GREEDY, n_bins, n_steps)
    got = host(q.quantize_rowwise(dev(x), 4, q.GREEDY, n_bins, n_steps))
    assert np.array_equal(got, ref)
    if n_steps == 0:
        assert np.array_equal(got, oracle.quantize_rowwise(x, 4, oracle.RANGE))


def test_greedy_on_ctr_and_quantizer_workload_shapes(q):
    """The d=16 Gaussian rows of the CTR one-hot workload and the d=64
    Gaussian/Laplace mixture rows of the quantizer workload, at the defaults
    (200 bins, 100 steps)."""
    for wid, rows in ((2, 20000), (5, 6000)):
        w = synth.workload(wid)
        x = synth.table_values_np(w, 0 if wid == 5 else int(np.argmax(w.rows)), 0, rows)
        for bits in (4, 8):
            ref = oracle.quantize_rowwise(x, bits, oracle.GREEDY, w.n_bins, w.n_steps)
            got = host(q.quantize_rowwise(dev(x), bits, q.GREEDY, w.n_bins, w.n_steps))
            assert np.array_equal(got, ref), (wid, bits)


# ---------------------------------------------------------------------------
# dequantize on arbitrary packed rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", [1, 2, 3, 5, 8, 16, 31, 32, 33, 63, 64, 65, 100, 128, 1000])
def test_dequantize_arbitrary_rows(q, dim, bits):
    """Random code bytes and random finite fp16 scale/bias (not produced by
    the quantizer) decode identically."""
    g = np.random.default_rng(3000 + dim + bits)
    S = oracle.row_stride(dim, bits)
    C = (dim * bits + 7) // 8
    rows = 2049
    packed = np.zeros((rows, S), np.uint8)
    packed[:, :C] = g.integers(0, 256, size=(rows, C), dtype=np.uint8)
    if bits == 4 and dim % 2:
        packed[:, C - 1] &= 0x0F
    prm = g.integers(0, 1 << 16, size=(rows, 2), dtype=np.uint32).astype(np.uint16)
    prm[(prm & 0x7C00) == 0x7C00] &= 0xBFFF  # keep finite
    packed[:, C:C + 4] = prm.view(np.uint8).reshape(rows, 4)
    y = host(q.dequantize(dev(packed), dim, bits))
    assert np.array_equal(y.view(np.uint32), oracle.dequantize(packed, dim, bits).view(np.uint32))


# ---------------------------------------------------------------------------
# normalized l2 error
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dim", [16, 64, 100])
def test_l2_error_matches_oracle(q, dim):
    g = np.random.default_rng(4000 + dim)
    x = special_rows(g, 50000 + 17, dim)
    for bits, mode in ((4, oracle.RANGE), (4, oracle.GREEDY), (8, oracle.RANGE)):
        packed = oracle.quantize_rowwise(x, bits, mode, 200, 100)
        ref = oracle.l2_error(x, packed, bits)
        got = q.l2_error(dev(x), dev(packed), bits)
        assert got["rows"] == ref["rows"]
        for k in ("mean_row", "sum_err2", "sum_x2"):
            assert abs(got[k] - ref[k]) <= 1e-12 * abs(ref[k]) + 1e-300, (k, got[k], ref[k])


# ---------------------------------------------------------------------------
# pooled lookup
# ---------------------------------------------------------------------------

def _run_bag(q, packed, bt, dim, bits, weights=None, total_rows=None, itype=np.int32):
    import torch
    idx = bt.indices.astype(itype)
    offs = bt.offsets.astype(itype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, dim, bits, dev(idx), dev(offs),
                        None if weights is None else dev(weights), err_count=err,
                        total_rows=total_rows)
    ref, absd, rerr = oracle.bag_forward(packed, bt.table_offsets, bt.B, dim, bits, idx, offs,
                                         weights, total_rows=total_rows)
    return host(out), int(host(err)[0]), ref, absd, rerr


def _table_for(w, bits, clip, rows):
    x = np.concatenate([synth.table_values_np(w, t, 0, rows[t]) for t in range(len(rows))])
    mode = oracle.GREEDY if clip == "greedy" else oracle.RANGE
    return x, oracle.quantize_rowwise(x, bits, mode, w.n_bins, w.n_steps)


def test_bag_tiny_workload(q):
    w = synth.workload(1)
    x, packed = _table_for(w, 4, "range", w.rows)
    bt = synth.batch(w)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, w.dim, 4)
    assert err == rerr == 0
    assert_pooled_close(got, ref, absd, "tiny")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_bag_multi_hot_weighted_scaled(q, bits, itype):
    """The multi-hot workload's shape (64 tables, d=128, bags of 1..64 ids,
    Zipf ids, U(0,1) weights) with 3000 rows per table and batch 300."""
    w = synth.scaled(synth.workload(4), rows=(3000,) * 64, batch=300)
    x, packed = _table_for(w, bits, "range", w.rows)
    bt = synth.batch(w, index_dtype=np.int64)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, w.dim, bits, bt.weights, itype=itype)
    assert err == rerr == 0
    assert_pooled_close(got, ref, absd, "multi-hot")


@pytest.mark.parametrize("wid,div", [(2, 1000), (3, 10000)])
def test_bag_one_hot_ctr_scaled(q, wid, div):
    """The CTR one-hot workloads' shapes (26 tables, pooling 1, Zipf ids) with
    row counts divided by `div`; the CTR-one-hot table is greedy-quantized."""
    w0 = synth.workload(wid)
    w = synth.scaled(w0, rows=[max(3, r // div) for r in w0.rows])
    x, packed = _table_for(w, 4, w.clip, w.rows)
    bt = synth.batch(w)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, w.dim, 4)
    assert err == rerr == 0
    assert_pooled_close(got, ref, absd, "one-hot %d" % wid)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", [1, 3, 16, 33, 64, 100, 128, 130, 513, 1000, 1024])
@pytest.mark.parametrize("weighted", [False, True])
def test_bag_dims_ragged_bags(q, dim, bits, weighted):
    g = np.random.default_rng(5000 + dim * 3 + bits + weighted)
    T, B = 3, 97
    rows = [1, 57, 300]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0  # keep the tolerance meaningful
    packed = oracle.quantize_rowwise(x, bits)
    lengths = g.integers(0, 71, size=T * B)
    lengths[::11] = 0
    offsets = np.concatenate([[0], np.cumsum(lengths)])
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lengths[gb]) for gb in range(T * B)])
    bt = synth.Batch(idx.astype(np.int32), offsets.astype(np.int32),
                     g.random(idx.size).astype(np.float32) if weighted else None,
                     np.concatenate([[0], np.cumsum(rows)]).astype(np.int64), B, T)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights)
    assert err == rerr == 0
    assert_pooled_close(got, ref, absd, "dim %d" % dim)
    empty = (lengths == 0).reshape(T, B).T
    assert np.all(got[empty] == 0) and not np.any(np.signbit(got[empty]))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", [16, 128])
def test_bag_long_and_boundary_lengths(q, dim, bits):
    """Bag lengths around the lookup's batch sizes (31..33, 63..65) and far
    past them (500, 1000), between empty and one-id bags."""
    g = np.random.default_rng(5500 + dim + bits)
    T, B = 2, 12
    rows = [700, 900]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, bits)
    lengths = np.array([0, 1, 500, 64, 65, 33, 31, 32, 1000, 2, 63, 0] * T)
    offsets = np.concatenate([[0], np.cumsum(lengths)])
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lengths[gb]) for gb in range(T * B)])
    bt = synth.Batch(idx.astype(np.int32), offsets.astype(np.int32), g.random(idx.size).astype(np.float32),
                     np.concatenate([[0], np.cumsum(rows)]).astype(np.int64), B, T)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights)
    assert err == rerr == 0
    assert_pooled_close(got, ref, absd, "long bags dim %d" % dim)


def test_bag_invalid_ids_and_offsets_are_skipped_and_counted(q):
    g = np.random.default_rng(6000)
    dim, bits, T, B = 64, 4, 4, 50
    rows = [100, 10, 1, 40]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, bits)
    lengths = g.integers(0, 12, size=T * B)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = np.concatenate([g.integers(-5, rows[gb // B] + 5, size=lengths[gb])
                          for gb in range(T * B)]).astype(np.int64)
    offsets[17] = offsets[16] - 1             # decreasing
    offsets[90] = offsets[-1] + 3             # past nnz
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    bt = synth.Batch(idx, offsets, g.random(idx.size).astype(np.float32), toff, B, T)
    for itype in (np.int32, np.int64):
        got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights, itype=itype)
        assert err == rerr and err > 20
        assert_pooled_close(got, ref, absd, "invalid")
    # a table whose row range leaves the packed buffer: every term of it skipped
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights,
                                         total_rows=sum(rows) - 1)
    assert err == rerr
    assert_pooled_close(got, ref, absd, "table out of range")
    assert np.all(got[:, 3, :] == 0)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dim", [16, 32, 64, 128, 256, 512, 1000])
def test_bag_invalid_ids_in_long_bags(q, dim, bits):
    """Invalid ids, bad offsets and a table out of range in multi-hot bags
    (mean length well above 8: the one-wave-per-run lookups), each counted
    exactly once."""
    print("invalid ids, long bags dim=%d bits=%d" % (dim, bits), flush=True)
    g = np.random.default_rng(6200 + dim + bits)
    T, B = 3, 70
    rows = [300, 20, 150]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, bits)
    lengths = g.integers(8, 90, size=T * B)
    lengths[::13] = 0
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = np.concatenate([g.integers(-3, rows[gb // B] + 3, size=lengths[gb])
                          for gb in range(T * B)]).astype(np.int64)
    offsets[40] = offsets[39] - 1             # decreasing
    offsets[150] = offsets[-1] + 7            # past nnz
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    bt = synth.Batch(idx, offsets, g.random(idx.size).astype(np.float32), toff, B, T)
    for itype in (np.int32, np.int64):
        got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights, itype=itype)
        assert err == rerr and err > 50, (err, rerr)
        assert_pooled_close(got, ref, absd, "invalid ids, long bags")
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits, bt.weights,
                                         total_rows=sum(rows) - 1)
    assert err == rerr, (err, rerr)
    assert_pooled_close(got, ref, absd, "long bags, table out of range")
    assert np.all(got[:, 2, :] == 0)


def test_bag_no_ids_and_single_bag(q):
    g = np.random.default_rng(6100)
    dim, bits = 128, 4
    x = special_rows(g, 20, dim)
    packed = oracle.quantize_rowwise(x, bits)
    toff = np.array([0, 20], np.int64)
    bt = synth.Batch(np.zeros(0, np.int32), np.zeros(9, np.int32), None, toff, 8, 1)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits)
    assert err == 0 and np.all(got == 0)
    bt = synth.Batch(np.arange(20, dtype=np.int32), np.array([0, 20], np.int32), None, toff, 1, 1)
    got, err, ref, absd, rerr = _run_bag(q, packed, bt, dim, bits)
    assert err == 0
    assert_pooled_close(got, ref, absd, "single bag")


def test_bag_weight_doubling_and_determinism(q):
    """out(2w) == 2 out(w) bitwise (power-of-two scaling is exact in every
    fp32 step) and two runs agree bitwise."""
    import torch
    w = synth.scaled(synth.workload(4), rows=(2000,) * 64, batch=128)
    x, packed = _table_for(w, 4, "range", w.rows)
    bt = synth.batch(w)
    args = (dev(packed), dev(bt.table_offsets), bt.B, w.dim, 4, dev(bt.indices), dev(bt.offsets))
    o1 = host(q.bag_forward(*args, weights=dev(bt.weights)))
    o2 = host(q.bag_forward(*args, weights=dev(bt.weights)))
    o3 = host(q.bag_forward(*args, weights=dev(bt.weights * np.float32(2.0))))
    torch.cuda.synchronize()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal((2 * o1).view(np.uint32), o3.view(np.uint32))


def test_bag_on_gpu_packed_table(q):
    """The lookup on the table the GPU quantizer packed (the path bench.py
    times) matches the oracle end to end."""
    w = synth.scaled(synth.workload(4), rows=(2500,) * 64, batch=200)
    x = np.concatenate([synth.table_values_np(w, t) for t in range(w.n_tables)])
    bt = synth.batch(w)
    for bits in (4, 8):
        gp = q.quantize_rowwise(dev(x), bits, q.RANGE)
        ref_packed = oracle.quantize_rowwise(x, bits)
        assert np.array_equal(host(gp), ref_packed)
        out = q.bag_forward(gp, dev(bt.table_offsets), bt.B, w.dim, bits, dev(bt.indices),
                            dev(bt.offsets), dev(bt.weights))
        ref, absd, _ = oracle.bag_forward(ref_packed, bt.table_offsets, bt.B, w.dim, bits,
                                          bt.indices, bt.offsets, bt.weights)
        assert_pooled_close(host(out), ref, absd, "gpu-packed %d" % bits)


def test_loaded_library_is_built_from_current_sources(q):
    """The library the GPU tests run was built from the kernel sources in
    this tree (a stale build is refused at load time)."""
    from int4_row_wise_amd import build as qbuild
    q.qemb.check_built_from_current_source(qbuild.LIB)
    assert qbuild.built_source_sha256() == qbuild.source_sha256()
