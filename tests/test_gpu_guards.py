"""Every writer of the library writes exactly its output and nothing else.

Each output is a view into a larger device buffer whose 4 KiB head and tail
(and, before the call, the output itself) hold a sentinel byte.  Every op
runs twice, once over the sentinel 0xA5 and once over 0x5A:
- the head and tail keep their sentinel (no write outside the output);
- the two outputs are identical byte for byte, so no byte of the output
  kept the sentinel it started with (every byte written), except where an
  op's contract leaves bytes alone (the record buffer past the last record,
  which must then still hold the sentinel).
Row strides, bag layouts and dims are chosen to reach each kernel and its
partial-row and ragged-tail stores (dims not a multiple of 4 or of a lane's
chunk, rows of 1..64 lanes, bags of every kernel's length regime).  Parity
of the values themselves is tested elsewhere; a few checks here compare
with the oracle where that is cheap.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from int4_row_wise_amd import synth
from tests.gpu_common import dev, host, require_gpu, special_rows

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINELS = (0xA5, 0x5A)


@pytest.fixture(scope="module")
def q():
    return require_gpu()


class Guarded:
    """A device tensor of `shape` and `dtype` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype, sentinel):
        import torch
        self.shape = tuple(shape)
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * torch.empty(0, dtype=dtype).element_size()
        self.sentinel = sentinel
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), sentinel, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(self.shape)

    def inner(self):
        import torch
        torch.cuda.synchronize()
        raw = host(self.raw)
        head, tail = raw[:GUARD], raw[GUARD + self.nbytes:]
        assert np.all(head == self.sentinel), "write before the output: %d bytes" % int(
            (head != self.sentinel).sum())
        assert np.all(tail == self.sentinel), "write after the output: %d bytes" % int(
            (tail != self.sentinel).sum())
        return raw[GUARD:GUARD + self.nbytes]


def twice(make, run):
    """run(outputs) over outputs made with each sentinel; returns the inner
    bytes of each output for both runs (guards checked)."""
    got = []
    for s in SENTINELS:
        outs = make(s)
        run(*[o.t for o in outs])
        got.append([o.inner() for o in outs])
    return got


def assert_all_written(got, what):
    for k, (a, b) in enumerate(zip(got[0], got[1])):
        diff = a != b
        assert not diff.any(), "%s output %d: %d bytes not written" % (what, k, int(diff.sum()))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dim", [1, 3, 33, 64, 100, 128, 513])
def test_quantizers_write_only_their_rows(q, bits, dim):
    import torch
    g = np.random.default_rng(700 + dim * 3 + bits)
    rows = 301
    x = special_rows(g, rows, dim)
    xd = dev(x)
    S = q.row_stride(dim, bits)
    for name, fn in (("range", lambda o: q.quantize_rowwise(xd, bits, q.RANGE, out=o)),
                     ("greedy", lambda o: q.quantize_rowwise(xd, bits, q.GREEDY, 40, 12, out=o)),
                     ("symmetric", lambda o: q.quantize_baseline(xd, bits, q.SYMMETRIC, out=o)),
                     ("percentile", lambda o: q.quantize_baseline(xd, bits, q.PERCENTILE, 0.9, out=o)),
                     ("aciq", lambda o: q.quantize_baseline(xd, bits, q.ACIQ, out=o))):
        got = twice(lambda s: [Guarded((rows, S), torch.uint8, s)], fn)
        assert_all_written(got, name)
        if name == "range":
            assert np.array_equal(got[0][0].reshape(rows, S), oracle.quantize_rowwise(x, bits))
    packed = dev(oracle.quantize_rowwise(x, bits))
    got = twice(lambda s: [Guarded((rows, dim), torch.float32, s)],
                lambda o: q.dequantize(packed, dim, bits, out=o))
    assert_all_written(got, "dequantize")


@pytest.mark.parametrize("dim", [1, 17, 64, 100, 128])
def test_codebook_writers(q, dim):
    import torch
    g = np.random.default_rng(800 + dim)
    rows = 257
    x = special_rows(g, rows, dim)
    x[np.abs(x) > 100] = 1.0
    xd = dev(x)
    S = q.codebook_row_stride(dim)
    got = twice(lambda s: [Guarded((rows, S), torch.uint8, s)], lambda o: q.quantize_codebook(xd, out=o))
    assert_all_written(got, "codebook quantize")
    cb = dev(got[0][0].reshape(rows, S))
    got = twice(lambda s: [Guarded((rows, dim), torch.float32, s)],
                lambda o: q.dequantize_codebook(cb, dim, out=o))
    assert_all_written(got, "codebook dequantize")
    # codebook lookup, short and long bags
    for lo, hi in ((0, 4), (20, 60)):
        T, B = 2, 70
        lens = g.integers(lo, hi + 1, size=T * B)
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        idx = g.integers(0, rows // 2, size=int(offs[-1])).astype(np.int32)
        toff = dev(np.array([0, rows // 2, 2 * (rows // 2)], np.int64))
        got = twice(lambda s: [Guarded((B, T, dim), torch.float32, s)],
                    lambda o: q.bag_forward_codebook(cb, toff, B, dim, dev(idx), dev(offs), out=o))
        assert_all_written(got, "codebook lookup %d..%d" % (lo, hi))


# (bits, dim, bag lengths lo..hi): each lookup kernel and its store paths --
# several bags per wave (d 16, 33, 1000 short), packed runs (d 64, 100
# short; INT2 d 97), chunked runs with bag sums in LDS (INT4 d 128, short
# and long), one wave per bag (INT8 d 100 and INT2 d 128 long: 8 lanes;
# d 512, 1000 long: wide rows)
LOOKUPS = [(4, 16, 0, 6), (4, 33, 0, 6), (8, 1000, 0, 4), (4, 64, 0, 12), (4, 100, 0, 12),
           (4, 128, 0, 12), (8, 100, 0, 12), (2, 97, 0, 12), (4, 128, 30, 70), (8, 100, 30, 70),
           (2, 128, 30, 70), (4, 512, 10, 40), (8, 1000, 10, 40), (4, 16, 30, 70)]


@pytest.mark.parametrize("bits,dim,lo,hi", LOOKUPS)
def test_lookup_writes_only_its_output(q, bits, dim, lo, hi):
    import torch
    g = np.random.default_rng(900 + dim + bits + lo)
    T, B = 3, 130
    rows = [40, 1, 300]
    x = special_rows(g, sum(rows), dim)
    x[np.abs(x) > 100] = 1.0
    packed = oracle.quantize_rowwise(x, bits)
    lens = g.integers(lo, hi + 1, size=T * B)
    lens[::9] = 0
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx = np.concatenate([g.integers(-1, rows[gb // B] + 1, size=lens[gb]) for gb in range(T * B)]
                         + [np.zeros(0, np.int64)]).astype(np.int32)
    w = g.random(idx.size).astype(np.float32)
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    args = (dev(packed), dev(toff), B, dim, bits, dev(idx), dev(offs), dev(w))
    got = twice(lambda s: [Guarded((B, T, dim), torch.float32, s), Guarded((1,), torch.int32, s)],
                lambda o, e: (e.zero_(), q.bag_forward(*args, out=o, err_count=e)))
    assert_all_written(got, "lookup")
    ref, absd, rerr = oracle.bag_forward(packed, toff, B, dim, bits, idx, offs, w)
    assert int(got[0][1].view(np.int32)[0]) == rerr
    out = got[0][0].view(np.float32).reshape(B, T, dim).astype(np.float64)
    assert np.all(np.abs(out - ref) <= 1e-5 * absd + 1e-6)


@pytest.mark.parametrize("T,dim", [(1, 16), (5, 33), (26, 64), (64, 128)])
def test_interaction_writes_only_its_output(q, T, dim):
    import torch
    g = np.random.default_rng(1000 + T + dim)
    B = 37
    dense = dev(g.standard_normal((B, dim)).astype(np.float32))
    pooled = dev(g.standard_normal((B, T, dim)).astype(np.float32))
    W = q.interaction_width(T, dim)
    got = twice(lambda s: [Guarded((B, W), torch.float32, s)],
                lambda o: q.dot_interaction(dense, pooled, out=o))
    assert_all_written(got, "interaction")


@pytest.mark.parametrize("n,dim", [(1, 1), (78, 33), (999, 128)])
def test_compression_writers(q, n, dim):
    import torch
    g = np.random.default_rng(1100 + n + dim)
    T = 3 if n % 3 == 0 else 1
    x = special_rows(g, n, dim)
    x[np.abs(x) > 1e4] = 0.5
    eb = np.array([1e-3, 1e-2, 0.0][:T], np.float32)
    xd, ebd = dev(x), dev(eb)
    cap = q.compress_bound(n, dim)
    wsb = max(q.compress_workspace_bytes(n), 16)
    got = twice(lambda s: [Guarded((cap,), torch.uint8, s), Guarded((n + 1,), torch.int64, s),
                           Guarded((wsb,), torch.uint8, s)],
                lambda o, f, w: q.compress_pooled(xd, ebd, T, out=o, offs=f, workspace=w))
    offs0, offs1 = got[0][1].view(np.int64), got[1][1].view(np.int64)
    assert np.array_equal(offs0, offs1)
    total = int(offs0[-1])
    assert 0 < total <= cap
    assert np.array_equal(got[0][0][:total], got[1][0][:total])
    # bytes past the last record are left alone
    for k, s in enumerate(SENTINELS):
        assert np.all(got[k][0][total:] == s)
    rbuf, roffs, _ = oracle.compress_pooled(x, eb)
    assert np.array_equal(offs0, roffs) and np.array_equal(got[0][0][:total], rbuf)
    buf, offs = dev(got[0][0][:total].copy()), dev(offs0.copy())
    got = twice(lambda s: [Guarded((n, dim), torch.float32, s), Guarded((1,), torch.int32, s)],
                lambda y, e: (e.zero_(), q.decompress_pooled(buf, offs, dim, ebd, y=y, err_count=e)))
    assert_all_written(got, "decompress")


def test_l2_writes_only_its_outputs(q):
    import torch
    g = np.random.default_rng(1200)
    x = special_rows(g, 999, 64)
    xd = dev(x)
    packed = dev(oracle.quantize_rowwise(x, 4))
    cb = q.quantize_codebook(xd)
    wsb = q.qemb.l2_error_workspace_bytes()
    for name, fn in (("l2", lambda w, o: q.l2_error(xd, packed, 4, workspace=w, out4=o)),
                     ("l2 codebook", lambda w, o: q.l2_error_codebook(xd, cb, workspace=w, out4=o))):
        got = twice(lambda s: [Guarded((wsb,), torch.uint8, s), Guarded((4,), torch.float64, s)], fn)
        assert np.array_equal(got[0][1], got[1][1]), name


def test_multi_hot_lookup_at_full_grid_writes_only_its_output(q):
    """The multi-hot workload's shape (64 tables, d=128, U{1..64} bags) with
    small tables: the grid of the full batch (16384 bags per table), the
    XCD block order included."""
    import torch
    w = synth.scaled(synth.workload(4), rows=(500,) * 64)
    x = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    packed = dev(oracle.quantize_rowwise(x, 4))
    bt = synth.batch(w)
    args = (packed, dev(bt.table_offsets), bt.B, w.dim, 4, dev(bt.indices), dev(bt.offsets), dev(bt.weights))
    got = twice(lambda s: [Guarded((bt.B, bt.T, w.dim), torch.float32, s)],
                lambda o: q.bag_forward(*args, out=o))
    assert_all_written(got, "multi-hot lookup")
