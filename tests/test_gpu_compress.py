"""GPU parity of the error-bounded compression of pooled vectors
("Avancées dans les recommandations en Deep Learning", scisimple page,
"Méthodes de Compression des Données", "Stratégies de Compression
Adaptative") against the CPU oracle.

Bars (integer and byte work): offsets and record bytes identical to the
oracle's; decompressed values bit-identical to the oracle's decoding of the
same records; malformed records counted and zeroed as the oracle does.  At
the multi-hot workload's full size (16384 x 64 vectors of d = 128) sampled
records are compared byte for byte and the bound is checked on every
element."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.gpu_common import dev, host, require_gpu, special_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    return require_gpu()


def _pooled(g, n, d):
    """Pooled-like vectors (sums of weighted rows) mixed with the special
    cases: zeros, -0, denormals, huge values, NaN / inf, grid values."""
    x = (g.standard_normal((n, d)) * 0.02 * np.sqrt(g.integers(1, 65, size=(n, 1)) / 3.0)).astype(np.float32)
    sp = special_rows(g, n, d)
    pick = g.random(n) < 0.3
    x[pick] = sp[pick]
    if n > 10:
        x[3] = 0.0
        x[4, ::2] = -0.0
        x[5] = np.float32(1e-41)
        x[6, d // 2] = np.float32(np.nan)
        x[7, 0] = np.float32(np.inf)
        x[8, -1] = np.float32(3e38)
        x[9] = (np.arange(d) % 15 - 7).astype(np.float32) * np.float32(0.5)
    return x


def _compare(q, x, T, ebs, what):
    import torch
    d = x.shape[1]
    ref_buf, ref_offs, ref_w = oracle.compress_pooled(x, ebs)
    buf, offs = q.compress_pooled(dev(x), dev(ebs), T=T)
    go = host(offs)
    assert np.array_equal(go, ref_offs), what + ": offsets"
    gb = host(buf)[: go[-1]]
    assert np.array_equal(gb, ref_buf), what + ": records"
    # the GPU decoder on the oracle's records, bit for bit
    y = host(q.decompress_pooled(dev(ref_buf) if ref_buf.size else torch.zeros(4, dtype=torch.uint8, device="cuda"),
                                 dev(ref_offs), d, dev(ebs), in_bytes=ref_buf.size))
    ry, bad = oracle.decompress_pooled(ref_buf, ref_offs, d, ebs)
    assert bad == 0
    assert np.array_equal(y.view(np.uint32), ry.view(np.uint32)), what + ": decoded"
    return ref_w


@pytest.mark.parametrize("d", [1, 2, 3, 16, 31, 63, 64, 65, 100, 128, 129, 200, 256, 500, 513, 1000, 1024])
def test_compress_matches_oracle(q, d):
    print("compress d=%d" % d, flush=True)
    g = np.random.default_rng(13000 + d)
    T = 3
    n = 3 * 64 + 37 if d <= 256 else 64 + 5  # several blocks and a ragged tail
    x = _pooled(g, n, d)
    ebs = np.array([1e-3, 0.05, 2.0], np.float32)
    w = _compare(q, x, T, ebs, "d=%d" % d)
    assert (w == oracle.RAW_WIDTH).any() and (w < oracle.RAW_WIDTH).any()


@pytest.mark.parametrize("n", [0, 1, 63, 64, 65, 128, 1000, 64 * 1024 + 3, 64 * 4096 + 65])
def test_compress_vector_counts(q, n):
    print("compress n=%d" % n, flush=True)
    g = np.random.default_rng(13100 + n)
    d, T = 128, 64 if n >= 64 else 1
    x = _pooled(g, n, d) if n else np.zeros((0, d), np.float32)
    ebs = (g.uniform(1e-4, 1e-2, size=T)).astype(np.float32)
    _compare(q, x, T, ebs, "n=%d" % n)


@pytest.mark.parametrize("d", [5, 64, 128, 300])
def test_arbitrary_bit_patterns(q, d):
    """Random float32 bit patterns (NaN payloads, infinities, denormals, every
    exponent) mixed with tame vectors, random bounds: records bit-exact."""
    g = np.random.default_rng(13700 + d)
    n, T = 300, 7
    x = g.integers(0, 2 ** 32, size=(n, d), dtype=np.uint64).astype(np.uint32).view(np.float32)
    tame = g.random(n) < 0.6
    x[tame] = (g.integers(-1000, 1001, size=(int(tame.sum()), d)) * 1e-3).astype(np.float32)
    ebs = np.exp(g.uniform(np.log(1e-6), np.log(10.0), size=T)).astype(np.float32)
    w = _compare(q, x, T, ebs, "bit patterns d=%d" % d)
    assert (w == oracle.RAW_WIDTH).any() and (w < oracle.RAW_WIDTH).any()


def test_bounds_that_force_verbatim(q):
    g = np.random.default_rng(13200)
    d, T = 64, 6
    x = _pooled(g, 6 * 50, d)
    ebs = np.array([0.0, -1.0, np.nan, np.inf, 3e38, 1e-30], np.float32)
    w = _compare(q, x, T, ebs, "special bounds")
    assert np.all(w.reshape(-1, T)[:, :5] == oracle.RAW_WIDTH)


def test_code_limit(q):
    """|q| < 2^30: q = -(2^30 - 64) is coded in 31 bits, q = -2^30 and
    +2^30 are stored verbatim (eb = 1, step 2, x = 2q exactly)."""
    lim = np.zeros((4, 32), np.float32)
    lim[0, 0] = np.float32(-(2.0 ** 31 - 128))
    lim[1, 0] = np.float32(-(2.0 ** 31))
    lim[2, 5] = np.float32(2.0 ** 31 - 128)
    lim[3, 31] = np.float32(2.0 ** 31)
    w = _compare(q, lim, 1, np.array([1.0], np.float32), "code limit")
    assert list(w) == [31, oracle.RAW_WIDTH, 31, oracle.RAW_WIDTH]


def test_adaptive_bounds_and_determinism(q):
    """The bound changes between calls (a looser one early in training, a
    tighter one later): each call matches the oracle under its own bounds,
    reusing the output, offsets and workspace; two identical calls agree."""
    import torch
    g = np.random.default_rng(13300)
    B, T, d = 40, 26, 64
    x = (g.standard_normal((B, T, d)) * 0.1).astype(np.float32)
    xd = dev(x)
    n = B * T
    out = torch.empty(q.compress_bound(n, d), dtype=torch.uint8, device="cuda")
    offs = torch.empty(n + 1, dtype=torch.int64, device="cuda")
    ws = torch.empty(q.compress_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    sizes = []
    r = g.uniform(0.5, 2.0, size=T)
    for scale in (1e-1, 1e-2, 1e-3, 1e-3):
        ebs = (scale * r).astype(np.float32)
        q.compress_pooled(xd, dev(ebs), out=out, offs=offs, workspace=ws)
        rb, ro, _ = oracle.compress_pooled(x, ebs)
        go = host(offs)
        assert np.array_equal(go, ro) and np.array_equal(host(out)[: go[-1]], rb)
        sizes.append(int(go[-1]))
    assert sizes[0] < sizes[1] < sizes[2] == sizes[3]  # tighter bounds, bigger payload


def test_malformed_records(q):
    import torch
    g = np.random.default_rng(13400)
    d = 48
    x = _pooled(g, 130, d)
    ebs = np.array([0.01], np.float32)
    rb, ro, _ = oracle.compress_pooled(x, ebs)
    o = ro.copy()
    o[10] = o[11] + 4                     # records 9, 10 out of order / wrong size
    o[50] = -8                            # records 49, 50 out of range
    b = rb.copy()
    b[o[70]:o[70] + 4] = np.frombuffer(np.uint32(40).tobytes(), np.uint8)   # header above 32
    o[-1] = rb.size + 16                  # last record past the buffer
    for cut in (rb.size, rb.size - 12):   # and a buffer shorter than its offsets say
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y = host(q.decompress_pooled(dev(b), dev(o), d, dev(ebs), err_count=err, in_bytes=cut))
        ry, bad = oracle.decompress_pooled(b[:cut], o, d, ebs)
        assert int(host(err)[0]) == bad >= 6
        assert np.array_equal(y.view(np.uint32), ry.view(np.uint32))


def test_round_trip_bound_on_gpu_records(q):
    """The GPU's own records decoded by the GPU: every element within its
    table's bound (checked in binary64, exact for these fp32 pairs), the
    verbatim vectors bit-exact."""
    g = np.random.default_rng(13500)
    B, T, d = 300, 8, 128
    x = _pooled(g, B * T, d)
    ebs = np.logspace(-5, 0, T).astype(np.float32)
    buf, offs = q.compress_pooled(dev(x), dev(ebs), T=T)
    y = host(q.decompress_pooled(buf, offs, d, dev(ebs)))
    e = np.tile(ebs, B)[:, None].astype(np.float64)
    fin = np.isfinite(x).all(axis=1)
    diff = np.abs(x[fin].astype(np.float64) - y[fin].astype(np.float64))
    assert np.all(diff <= np.broadcast_to(e, x.shape)[fin])
    assert np.array_equal(y[~fin].view(np.uint32), x[~fin].view(np.uint32))


def test_compress_full_multi_hot_output(q):
    """16384 x 64 pooled vectors of d = 128 (the multi-hot workload's output
    shape, values like sums of 1..64 weighted rows), per-table bounds of 1 %
    of the table's standard deviation: 2000 sampled records byte for byte
    against the oracle (records are independent, so the oracle compresses
    just the sampled vectors) with their offset differences equal to the
    oracle's record sizes, and the bound on every element of the GPU round
    trip."""
    import torch
    print("compress full size", flush=True)
    B, T, d = 16384, 64, 128
    gen = torch.Generator(device="cuda").manual_seed(13600)
    lens = torch.randint(1, 65, (B, T, 1), device="cuda", generator=gen).float()
    x = torch.randn((B, T, d), device="cuda", generator=gen) * 0.02 * torch.sqrt(lens / 3.0)
    ebs = (0.01 * x.std(dim=(0, 2))).float().contiguous()
    buf, offs = q.compress_pooled(x, ebs)
    y = q.decompress_pooled(buf, offs, d, ebs)
    diff = (x.double() - y.view(B, T, d).double()).abs()
    assert bool((diff <= ebs.double().view(1, T, 1)).all())
    go = host(offs)
    hb = host(buf[: int(go[-1])])
    g = np.random.default_rng(13601)
    vs = np.sort(g.choice(B * T, size=2000, replace=False))
    xs = x.view(B * T, d)[torch.from_numpy(vs).cuda()].cpu().numpy()
    ebh = host(ebs)
    for k, v in enumerate(vs):
        rb, ro, _ = oracle.compress_pooled(xs[k:k + 1], ebh[v % T: v % T + 1])
        assert go[v + 1] - go[v] == ro[1]
        assert np.array_equal(hb[go[v]: go[v + 1]], rb), v
    ratio = B * T * d * 4 / go[-1]
    print("compression ratio %.2f" % ratio, flush=True)
    assert ratio > 2.5
