"""Pins of the oracle's error-bounded compression of pooled embeddings
("Avancées dans les recommandations en Deep Learning", scisimple page,
"Méthodes de Compression des Données": a lossy method whose reconstruction
stays within a user-set maximum error; "Stratégies de Compression
Adaptative": one bound per table).

Each check ties the oracle to something other than its own code:
hand-derived records (tests/golden/compress_tiny.json); the bound itself,
checked in exact rational arithmetic; verbatim vectors bit for bit; the
packed stream read back with numpy's bit unpacking, which must give codes
of exactly the recorded width (no narrower width fits); record sizes in
closed form; the nearest-code property of every quantized element; and the
decoder's handling of malformed records.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "compress_tiny.json")


def _x_from_bits(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def _records(buf, offs):
    return [bytes(buf[offs[v]:offs[v + 1]]) for v in range(offs.size - 1)]


def _np_codes(buf, offs, d):
    """Header and codes of each record, read with numpy's bit unpacking."""
    out = []
    for v in range(offs.size - 1):
        rec = buf[offs[v]:offs[v + 1]]
        w = int(np.frombuffer(rec[:4].tobytes(), "<u4")[0])
        if w == oracle.RAW_WIDTH:
            out.append((w, None))
            continue
        bits = np.unpackbits(rec[4:], bitorder="little")[: d * w].reshape(d, w) if w else np.zeros((d, 0))
        u = (bits.astype(np.uint64) << np.arange(w, dtype=np.uint64)).sum(axis=1) if w else np.zeros(d, np.uint64)
        out.append((w, u.astype(np.int64)))
    return out


def _unzig(u):
    return np.where(u % 2 == 0, u // 2, -(u + 1) // 2)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_records(case):
    d, T = case["d"], case["T"]
    x = _x_from_bits(case["x_bits"]).reshape(-1, T, d)
    eb = np.array(case["eb"], np.float32)
    buf, offs, widths = oracle.compress_pooled(x, eb)
    assert list(widths) == case["w"]
    assert [r.hex() for r in _records(buf, offs)] == case["record_hex"]
    y, bad = oracle.decompress_pooled(buf, offs, d, eb)
    assert bad == 0
    if "y" in case:
        assert np.array_equal(y.reshape(-1), np.array(case["y"], np.float32))
        assert not np.any(np.signbit(y[np.asarray(widths) != oracle.RAW_WIDTH]) & (y[np.asarray(widths) != oracle.RAW_WIDTH] == 0))
    raw = np.asarray(widths) == oracle.RAW_WIDTH
    assert np.array_equal(y[raw].view(np.uint32), x.reshape(-1, d)[raw].view(np.uint32))
    if "u" in case:
        (w, u), = _np_codes(buf, offs, d)
        assert list(u) == case["u"] and list(_unzig(u)) == case["q"]


def _vectors(g, n, d, scale):
    x = g.standard_normal((n, d)).astype(np.float32) * np.float32(scale)
    x[::7] *= np.float32(1000.0)          # wide vectors
    x[1::11] = 0.0                        # all-zero vectors
    x[2::13, : max(1, d // 3)] = -0.0
    return x


@pytest.mark.parametrize("d", [1, 3, 16, 31, 64, 128, 200])
@pytest.mark.parametrize("eb", [1e-6, 1e-3, 0.05, 1.0, 1e6])
def test_bound_holds_exactly(d, eb):
    g = np.random.default_rng(int(d * 1000 + np.log10(eb) * 7 + 50))
    T = 3
    x = _vectors(g, 60, d, 1.0).reshape(20, T, d)
    ebs = np.array([eb, eb * 3.0, eb / 7.0], np.float32)
    buf, offs, widths = oracle.compress_pooled(x, ebs)
    y, bad = oracle.decompress_pooled(buf, offs, d, ebs)
    assert bad == 0
    xf = x.reshape(-1, d)
    for v in range(xf.shape[0]):
        e = Fraction(float(ebs[v % T]))
        for i in range(d):
            assert abs(Fraction(float(xf[v, i])) - Fraction(float(y[v, i]))) <= e, (v, i)
    raw = widths == oracle.RAW_WIDTH
    assert np.array_equal(y[raw].view(np.uint32), xf[raw].view(np.uint32))


@pytest.mark.parametrize("d", [1, 5, 32, 33, 128, 1000])
def test_widths_minimal_sizes_closed_form_codes_nearest(d):
    g = np.random.default_rng(700 + d)
    T = 2
    x = _vectors(g, 40, d, 3.0).reshape(20, T, d)
    ebs = np.array([0.01, 0.2], np.float32)
    buf, offs, widths = oracle.compress_pooled(x, ebs)
    xf = x.reshape(-1, d)
    assert offs[0] == 0 and buf.size == offs[-1] <= oracle.compress_bound(xf.shape[0], d)
    for v, (w, u) in enumerate(_np_codes(buf, offs, d)):
        assert w == widths[v]
        size = 4 + 4 * d if w == oracle.RAW_WIDTH else 4 + 4 * ((d * w + 31) // 32)
        assert offs[v + 1] - offs[v] == size
        if w == oracle.RAW_WIDTH:
            continue
        assert 0 <= w <= 31
        if w:
            assert int(u.max()) >> (w - 1) == 1  # the largest code needs all w bits
        else:
            assert not u.any()
        # every code is a nearest bin of x / step: no neighbour is closer
        step = Fraction(2) * Fraction(float(ebs[v % T]))
        q = _unzig(u)
        for i in range(d):
            t = Fraction(float(xf[v, i])) / step
            assert abs(t - int(q[i])) <= Fraction(1, 2) + Fraction(1, 1 << 20), (v, i)


def test_verbatim_cases():
    d = 8
    x = np.ones((6, d), np.float32)
    x[0, 3] = np.inf
    x[1, 0] = -np.inf
    x[2, 5] = np.float32(np.nan)
    x[3, 1] = np.float32(3e9)       # |x / step| >= 2^30 at eb = 1
    x[4] = 1e-40                     # denormals, coded (w = 0 at eb = 1)
    x[5] = 0.75
    for ebs, raw_expected in (([1.0], [1, 1, 1, 1, 0, 0]), ([0.0], [1] * 6), ([-1.0], [1] * 6),
                              ([np.nan], [1] * 6), ([np.inf], [1] * 6), ([3e38], [1] * 6)):
        e = np.array(ebs, np.float32)
        buf, offs, widths = oracle.compress_pooled(x, e)
        assert list((widths == oracle.RAW_WIDTH).astype(int)) == raw_expected, ebs
        y, bad = oracle.decompress_pooled(buf, offs, d, e)
        raw = widths == oracle.RAW_WIDTH
        assert bad == 0 and np.array_equal(y[raw].view(np.uint32), x[raw].view(np.uint32))
    # eb = 1: 0.75 -> q = rint(0.375) = 0, |0.75 - 0| <= 1
    buf, offs, widths = oracle.compress_pooled(x, np.array([1.0], np.float32))
    assert widths[5] == 0 and widths[4] == 0
    # the code limit |q| < 2^30: q = -(2^30 - 64) (the largest float below the
    # limit) is coded in 31 bits, q = -2^30 is not (step 2: x = 2q exactly)
    lim = np.zeros((2, 32), np.float32)
    lim[0, 0] = np.float32(-(2.0 ** 31 - 128))
    lim[1, 0] = np.float32(-(2.0 ** 31))
    buf, offs, widths = oracle.compress_pooled(lim, np.array([1.0], np.float32))
    assert list(widths) == [31, oracle.RAW_WIDTH]
    assert list(np.diff(offs)) == [4 + 4 * 31, 4 + 4 * 32]


def test_constant_grid_compression_ratio():
    """Values on the bin grid in [-7, 7] steps: codes up to 14 need 4 bits,
    so a d = 128 vector takes 4 + 64 bytes against 512 raw."""
    d = 128
    step = np.float32(0.5)
    q = (np.arange(d) % 15) - 7
    x = (q.astype(np.float32) * step)[None, None, :]
    buf, offs, widths = oracle.compress_pooled(x, np.array([0.25], np.float32))
    assert widths[0] == 4 and offs[-1] == 68
    y, _ = oracle.decompress_pooled(buf, offs, d, np.array([0.25], np.float32))
    assert np.array_equal(y[0], x[0, 0])


def test_malformed_records_are_counted_and_zeroed():
    g = np.random.default_rng(5)
    d = 16
    x = g.standard_normal((5, d)).astype(np.float32)
    eb = np.array([0.01], np.float32)
    buf, offs, widths = oracle.compress_pooled(x, eb)
    good, _ = oracle.decompress_pooled(buf, offs, d, eb)
    o = offs.copy()
    o[2] = o[3] + 4               # records 1 and 2: out of order / wrong size
    b = buf.copy()
    b[o[4]:o[4] + 4] = np.frombuffer(np.uint32(33).tobytes(), np.uint8)  # header > 32
    y, bad = oracle.decompress_pooled(b, o, d, eb)
    assert bad == 3
    assert np.all(y[[1, 2, 4]] == 0) and np.array_equal(y[[0, 3]], good[[0, 3]])
    o2 = offs.copy()
    o2[-1] = buf.size + 8         # past the buffer
    y, bad = oracle.decompress_pooled(buf, o2, d, eb)
    assert bad == 1 and np.all(y[-1] == 0)


def test_empty():
    buf, offs, widths = oracle.compress_pooled(np.zeros((0, 3, 8), np.float32), np.ones(3, np.float32))
    assert buf.size == 0 and list(offs) == [0] and widths.size == 0


def test_properties_over_arbitrary_bit_patterns():
    """Any float32 bit patterns (NaN, inf, denormals included) and any bound:
    every coded element within its bound (exact rationals), verbatim vectors
    bit for bit, each coded record at the minimal width, sizes in closed
    form, and the decoder's own records decode with no error."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=150, deadline=None, derandomize=True)
    @given(st.integers(1, 40), st.integers(1, 4), st.integers(1, 5), st.data())
    def check(d, T, B, data):
        bits = data.draw(st.lists(st.integers(0, 2 ** 32 - 1), min_size=B * T * d, max_size=B * T * d))
        x = np.array(bits, dtype=np.uint32).view(np.float32).reshape(B, T, d)
        # mostly tame values: keep a random subset of the raw patterns, scale the rest
        tame = data.draw(st.lists(st.booleans(), min_size=B * T, max_size=B * T))
        xf = x.reshape(-1, d)
        for v, t in enumerate(tame):
            if t:
                xf[v] = (np.array(bits[v * d:(v + 1) * d], np.int64) % 2001 - 1000).astype(np.float32) * np.float32(1e-3)
        ebs = np.array(data.draw(st.lists(st.floats(float(np.float32(1e-6)), 10.0, width=32), min_size=T, max_size=T)), np.float32)
        buf, offs, widths = oracle.compress_pooled(x, ebs)
        y, bad = oracle.decompress_pooled(buf, offs, d, ebs)
        assert bad == 0
        for v, (w, u) in enumerate(_np_codes(buf, offs, d)):
            size = 4 + 4 * d if w == oracle.RAW_WIDTH else 4 + 4 * ((d * w + 31) // 32)
            assert offs[v + 1] - offs[v] == size
            if w == oracle.RAW_WIDTH:
                assert np.array_equal(y[v].view(np.uint32), xf[v].view(np.uint32))
                continue
            assert (w == 0 and not u.any()) or int(u.max()) >> (w - 1) == 1
            e = Fraction(float(ebs[v % T]))
            for i in range(d):
                assert abs(Fraction(float(xf[v, i])) - Fraction(float(y[v, i]))) <= e

    check()
