"""GPU parity of the pooled lookup on bags of a few to a few tens of ids over
rows of 4 to 8 lanes of 16 codes (INT4 d 49..128, INT8 d 33..128, INT2 d
49..128; INT4 rows of d 127 and 128 take these runs only for one id per bag
on average, and the chunked runs of tests/test_gpu_seg.py otherwise, so
those cases here check that kernel too): the lookup packs runs of 64 consecutive bags of a table into full
id batches, splits each run's ids evenly over the wave's row groups and
completes bags cut by those splits at the end of the run.  The cases put
bags across the splits (long bags between short ones, a bag spanning every
group), runs of empty bags, partial runs (batch sizes that are not a
multiple of 64) and many small tables, with every row-layout variant
(scale/bias after the last lane's codes, on a 4-byte boundary or not).

Bars as everywhere: pooled outputs within 1e-5 * sum|terms| + 1e-6 of the
oracle (the fp64 pooled lookup of the oracle-packed rows), error counts
exact, empty bags +0.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from int4_row_wise_amd import synth
from tests.gpu_common import assert_pooled_close, dev, host, require_gpu, special_rows

pytestmark = pytest.mark.gpu

# (bits, dim): 4 and 8 lanes per row; the scale/bias right after the last
# lane's codes (INT4 d 64, 128), 4-byte aligned after a partial lane
# (INT4 120, INT8 100, INT2 128) or not aligned (INT4 49, 100; INT8 33;
# INT2 97)
SHAPES = [(4, 49), (4, 64), (4, 100), (4, 120), (4, 128), (8, 33), (8, 64), (8, 100), (8, 128),
          (2, 64), (2, 97), (2, 128)]


@pytest.fixture(scope="module")
def q():
    return require_gpu()


def _lengths(g, kind, n):
    if kind == "short":
        lens = g.integers(0, 17, size=n)
        lens[::7] = 0
    elif kind == "one":
        lens = np.ones(n, np.int64)
    elif kind == "spans":
        # mostly short bags, a few of 100..300 ids that run across several
        # of a run's group chunks, and some runs of empty bags
        lens = np.where(g.random(n) < 0.03, g.integers(100, 300, size=n), g.integers(0, 6, size=n))
        lens[40:110] = 0
    elif kind == "mean24":
        lens = g.integers(16, 32, size=n)
    else:
        raise ValueError(kind)
    return lens.astype(np.int64)


def _case(g, bits, dim, T, B, rows, lens, weighted):
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0  # keep the tolerance meaningful
    packed = oracle.quantize_rowwise(x, bits)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lens[gb]) for gb in range(T * B)]
                         + [np.zeros(0, np.int64)]).astype(np.int64)
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    w = g.random(idx.size).astype(np.float32) if weighted else None
    return packed, synth.Batch(idx, offs, w, toff, B, T)


def _check(q, packed, bt, dim, bits, itype, what, total_rows=None):
    import torch
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = bt.indices.astype(itype)
    offs = bt.offsets.astype(itype)
    out = host(q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, dim, bits, dev(idx), dev(offs),
                             None if bt.weights is None else dev(bt.weights), err_count=err,
                             total_rows=total_rows))
    ref, absd, rerr = oracle.bag_forward(packed, bt.table_offsets, bt.B, dim, bits, idx, offs, bt.weights,
                                         total_rows=total_rows)
    gerr = int(host(err)[0])
    assert gerr == rerr, (what, gerr, rerr)
    assert_pooled_close(out, ref, absd, what)
    return out


def _mean_len(bt):
    return -(-int(bt.offsets[-1]) // (bt.T * bt.B))


# bags of 16..32 ids take the packed runs for INT4 rows only
RUN_CASES = [(bits, dim, kind) for bits, dim in SHAPES for kind in ("short", "one", "spans", "mean24")
             if kind != "mean24" or bits == 4]


@pytest.mark.parametrize("bits,dim,kind", RUN_CASES)
def test_packed_runs_match_oracle(q, bits, dim, kind):
    print("packed runs bits=%d dim=%d %s" % (bits, dim, kind), flush=True)
    g = np.random.default_rng(9100 + 7 * dim + bits + len(kind))
    T, B = 3, 150
    rows = [1, 70, 400]
    for weighted in (True, False):
        packed, bt = _case(g, bits, dim, T, B, rows, _lengths(g, kind, T * B), weighted)
        assert _mean_len(bt) <= (24 if bits == 4 else 16)
        for itype in (np.int32, np.int64):
            out = _check(q, packed, bt, dim, bits, itype, "%s d=%d bits=%d w=%d %s" % (
                kind, dim, bits, weighted, itype.__name__))
        lens = np.diff(bt.offsets).reshape(T, B).T
        assert np.all(out[lens == 0] == 0) and not np.any(np.signbit(out[lens == 0]))


@pytest.mark.parametrize("bits,dim", [(4, 128), (8, 64), (2, 128)])
def test_packed_one_bag_across_every_group(q, bits, dim):
    """A run whose ids are almost all in one bag (it spans every group's
    chunk: the first group adds all middle pieces and the last piece), with
    short bags before and after it, and a run of a single bag of 12 ids
    (spread over several groups)."""
    g = np.random.default_rng(9300 + dim + bits)
    T, B = 2, 64
    rows = [500, 300]
    lens = np.zeros(T * B, np.int64)
    lens[:64] = g.integers(0, 3, size=64)
    lens[10] = 700
    lens[64 + 63] = 1000  # the last bag of the last run
    packed, bt = _case(g, bits, dim, T, B, rows, lens, True)
    assert _mean_len(bt) <= 16
    _check(q, packed, bt, dim, bits, np.int32, "one bag across every group")
    packed, bt = _case(g, bits, dim, 1, 1, [50], np.array([12]), True)
    _check(q, packed, bt, dim, bits, np.int32, "a run of one bag")


@pytest.mark.parametrize("bits,dim", [(4, 64), (4, 128), (8, 100), (2, 97)])
def test_packed_invalid_ids_offsets_and_tables(q, bits, dim):
    """Ids outside their table, decreasing offsets, offsets past nnz and a
    table outside the packed buffer: each skipped and counted exactly once."""
    g = np.random.default_rng(9400 + dim + bits)
    T, B = 4, 90
    rows = [100, 10, 1, 40]
    packed, bt = _case(g, bits, dim, T, B, rows, _lengths(g, "short", T * B), True)
    bad = g.random(bt.indices.size) < 0.1
    bt.indices[bad] = g.choice([-1, -5, -(1 << 31), 1 << 20], size=int(bad.sum()))
    for t in range(T):  # ids just past each table
        s0, s1 = bt.offsets[t * B], bt.offsets[(t + 1) * B]
        bt.indices[s0:s1:9] = rows[t]
    bt.offsets[17] = bt.offsets[16] - 1
    bt.offsets[200] = bt.offsets[-1] + 3
    for itype in (np.int32, np.int64):
        _check(q, packed, bt, dim, bits, itype, "invalid %s" % itype.__name__)
    out = _check(q, packed, bt, dim, bits, np.int64, "table out of range", total_rows=sum(rows) - 1)
    assert np.all(out[:, 3, :] == 0)
    out = _check(q, packed, bt, dim, bits, np.int32, "no rows", total_rows=0)
    assert np.all(out == 0)


@pytest.mark.parametrize("bits,dim", [(4, 128), (8, 64)])
def test_packed_batch_shapes(q, bits, dim):
    """Batch sizes around the 64-bag runs (1, 63, 64, 65, 200) and many
    tables (70 tables of 3 rows, batch 5)."""
    g = np.random.default_rng(9500 + dim + bits)
    for T, B in ((2, 1), (3, 63), (2, 64), (2, 65), (1, 200), (70, 5)):
        rows = [3] * T if T > 3 else [50, 3, 20][:T]
        packed, bt = _case(g, bits, dim, T, B, rows, _lengths(g, "short", T * B), True)
        _check(q, packed, bt, dim, bits, np.int32, "T=%d B=%d" % (T, B))

