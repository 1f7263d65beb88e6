"""GPU parity of the pooled lookup over rows of 128 codes in 8 lanes (INT4
rows of 64 code bytes, d 127 and 128; INT2 rows of 32, d 125 and 128) for
bags of two or more ids on average: the lookup cuts runs of 24
consecutive bags of a table into equal chunks, one per row group of the
wave, keeps each bag's sum in LDS and writes the run's rows at its end.
The cases put bag ends on and off the chunk boundaries, bags longer than a
chunk (several groups hold pieces of them), runs of empty bags, partial
runs (batch sizes that are not a multiple of 24), runs whose CSR ranges do
not follow one another (invalid offsets: those runs are walked one bag at a
time), ids outside their table, int32 and int64 ids, weighted and plain
sums.

Bars as everywhere: pooled outputs within 1e-5 * sum|terms| + 1e-6 of the
oracle (the fp64 pooled lookup of the oracle-packed rows), error counts
exact, empty bags +0, two calls bit-identical.
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


def _lengths(g, kind, n):
    if kind == "mix":
        lens = g.integers(0, 71, size=n)
    elif kind == "short":
        lens = g.integers(1, 5, size=n)  # mean 2.5: the smallest mean that takes this kernel
    elif kind == "long":
        lens = g.integers(100, 401, size=n)
    elif kind == "threes":
        lens = np.full(n, 3)  # 24 bags of 3: a bag ends on every chunk boundary
    elif kind == "eights":
        lens = np.full(n, 8)
    elif kind == "spanning":
        # short bags with a few of 1000..3000 ids, longer than a group's chunk
        lens = np.where(g.random(n) < 0.02, g.integers(1000, 3001, size=n), g.integers(1, 8, size=n))
    elif kind == "empties":
        lens = g.integers(0, 9, size=n)
        lens[30:80] = 0
        lens[::5] = 0
    else:
        raise ValueError(kind)
    return lens.astype(np.int64)


def _case(g, dim, T, B, rows, lens, weighted, bits=4):
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0  # keep the tolerance meaningful
    packed = oracle.quantize_rowwise(x, bits)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lens[gb]) for gb in range(T * B)]
                         + [np.zeros(0, np.int64)]).astype(np.int64)
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    w = g.random(idx.size).astype(np.float32) if weighted else None
    return packed, synth.Batch(idx, offs, w, toff, B, T)


def _check(q, packed, bt, dim, itype, what, total_rows=None, bits=4):
    import torch
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = bt.indices.astype(itype)
    offs = bt.offsets.astype(itype)
    call = lambda: host(q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, dim, bits, dev(idx), dev(offs),
                                      None if bt.weights is None else dev(bt.weights), err_count=err,
                                      total_rows=total_rows))
    out = call()
    ref, absd, rerr = oracle.bag_forward(packed, bt.table_offsets, bt.B, dim, bits, idx, offs, bt.weights,
                                         total_rows=total_rows)
    gerr = int(host(err)[0])
    assert gerr == rerr, (what, gerr, rerr)
    assert_pooled_close(out, ref, absd, what)
    assert np.array_equal(out.view(np.uint32), call().view(np.uint32)), what + ": not repeatable"
    return out


SHAPES = [(4, 127), (4, 128), (2, 125), (2, 128)]


@pytest.mark.parametrize("bits,dim", SHAPES)
@pytest.mark.parametrize("kind", ["mix", "short", "long", "threes", "eights", "spanning", "empties"])
def test_chunked_runs_match_oracle(q, bits, dim, kind):
    print("chunked runs bits=%d dim=%d %s" % (bits, dim, kind), flush=True)
    g = np.random.default_rng(9600 + dim + 7 * bits + 13 * len(kind))
    T, B = 3, 150
    rows = [1, 70, 400]
    for weighted in (True, False):
        packed, bt = _case(g, dim, T, B, rows, _lengths(g, kind, T * B), weighted, bits)
        assert int(bt.offsets[-1]) >= 2 * T * B  # two or more ids per bag on average
        for itype in (np.int32, np.int64):
            out = _check(q, packed, bt, dim, itype, "%s bits=%d d=%d w=%d %s" % (
                kind, bits, dim, weighted, itype.__name__), bits=bits)
        lens = np.diff(bt.offsets).reshape(T, B).T
        assert np.all(out[lens == 0] == 0) and not np.any(np.signbit(out[lens == 0]))


@pytest.mark.parametrize("bits", [4, 2])
def test_chunked_runs_one_bag_across_every_group(q, bits):
    """A run of one bag, runs whose ids are almost all in one bag (it spans
    every group's chunk), and a last run of 7 bags."""
    g = np.random.default_rng(9700 + bits)
    packed, bt = _case(g, 128, 1, 1, [50], np.array([700]), True, bits)
    _check(q, packed, bt, 128, np.int32, "one bag of 700", bits=bits)
    T, B = 2, 55
    lens = np.full(T * B, 2, np.int64)
    lens[5] = 2500
    lens[B + 30] = 1200
    lens[T * B - 1] = 900  # the last bag of the last, partial run
    packed, bt = _case(g, 128, T, B, [500, 300], lens, True, bits)
    _check(q, packed, bt, 128, np.int32, "bags across every group", bits=bits)
    _check(q, packed, bt, 128, np.int64, "bags across every group, int64 ids", bits=bits)


@pytest.mark.parametrize("bits", [4, 2])
def test_chunked_runs_starting_off_the_8_id_grid(q, bits):
    """Runs whose first CSR position takes every value mod 8 and whose first
    bag (1000 ids) covers the first chunks entirely: the chunks are counted
    from the 8-id boundary below the run, so group 0's chunk starts before
    the run and holds no bag end (the case where the slot count to the
    chunk's 'no end' marker must not overflow)."""
    g = np.random.default_rng(9750 + bits)
    runs = 9
    lens = []
    pos = 0
    for r in range(runs):
        run = [1000] + [2] * 22
        pos += sum(run)
        last = 2 + ((r + 1 - (pos + 2)) % 8)  # the next run starts at position r + 1 (mod 8)
        run.append(last)
        pos += last
        lens += run
    lens = np.array(lens, np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)])[::24][:runs]
    assert [int(x) % 8 for x in starts] == [0, 1, 2, 3, 4, 5, 6, 7, 0]
    packed, bt = _case(g, 128, 1, lens.size, [300], lens, True, bits)
    for itype in (np.int32, np.int64):
        _check(q, packed, bt, 128, itype, "runs off the 8-id grid, %s" % itype.__name__, bits=bits)


@pytest.mark.parametrize("bits,dim", SHAPES)
def test_chunked_runs_invalid_ids_offsets_and_tables(q, bits, dim):
    """Ids outside their table, decreasing offsets, offsets past nnz and a
    table outside the packed buffer: each skipped and counted exactly once;
    runs with an invalid bag are walked one bag at a time."""
    g = np.random.default_rng(9800 + dim + bits)
    T, B = 4, 90
    rows = [100, 10, 1, 40]
    packed, bt = _case(g, dim, T, B, rows, _lengths(g, "mix", T * B), True, bits)
    bad = g.random(bt.indices.size) < 0.1
    bt.indices[bad] = g.choice([-1, -5, -(1 << 31), 1 << 20], size=int(bad.sum()))
    for t in range(T):  # ids just past each table
        s0, s1 = bt.offsets[t * B], bt.offsets[(t + 1) * B]
        bt.indices[s0:s1:9] = rows[t]
    offs = bt.offsets.copy()
    offs[7] = offs[8] + 3        # bag 6 ends past bag 7's start; bag 7 ends before it starts
    offs[100] = offs[-1] + 10    # bags 99 and 100 run past nnz
    bt = synth.Batch(bt.indices, offs, bt.weights, bt.table_offsets, B, T)
    for itype in (np.int32, np.int64):
        _check(q, packed, bt, dim, itype, "invalid ids and offsets bits=%d d=%d %s" % (bits, dim, itype.__name__),
               bits=bits)
    # the last table's rows lie past the packed buffer: every id of it is counted
    _check(q, packed, bt, dim, np.int32, "table outside the buffer", total_rows=120, bits=bits)
