"""Seeded synthetic inputs shaped like CTR embedding workloads.

This module only draws random inputs: table values, row counts, bag lengths,
indices and per-index weights.  It holds none of the quantization or lookup
arithmetic, and both the HIP path and the CPU oracle are fed from it.

The pages measure on Criteo Kaggle / Terabyte, Avazu and a production ranking
model (DQRM repository page, result tables; "Post-Training 4-bit Quantization
on Embedding Tables", abstract); none of those datasets is available here, so
these generators stand in for them with the shapes of the five workloads
below (sizes, value distributions, Zipf-skewed ids, multi-hot bag lengths).

Determinism: every draw comes from numpy's PCG64 seeded by a SeedSequence
keyed on (workload, stream, table, chunk), or, for table values generated on
the GPU, from torch's generator seeded by the same key; values are drawn in
fixed chunks of 2^20 rows so they do not depend on memory or chunk size.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

CHUNK_ROWS = 1 << 20

# stream ids of the seed key
S_VALUES, S_INDICES, S_LENGTHS, S_WEIGHTS, S_ROWCOUNTS = 0, 1, 2, 3, 4


def rng(workload: int, stream: int, table: int = 0, chunk: int = 0, seed: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(workload, stream, table, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def torch_seed(workload: int, stream: int, table: int = 0, chunk: int = 0, seed: int = 0) -> int:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(workload, stream, table, chunk))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


@dataclasses.dataclass(frozen=True)
class Values:
    """Distribution of table values.

    kind: "normal" (N(0, sigma)); "outliers" (N(0, sigma) where each element
    independently, with probability p_out, is replaced by +/-10 sigma with a
    uniform sign); "mixture" (each element independently from Laplace(0,
    lap_scale) with probability p_mix, else N(0, sigma)).
    """
    kind: str = "normal"
    sigma: float = 0.02
    p_out: float = 0.001
    out_mult: float = 10.0
    p_mix: float = 0.01
    lap_scale: float = 0.2


@dataclasses.dataclass(frozen=True)
class Workload:
    id: int
    name: str
    rows: tuple            # rows per table
    dim: int
    values: Values
    bits: tuple            # quantized widths exercised
    clip: str              # "range" or "greedy" (quantizer used for the lookup table)
    batch: int
    pooling: str           # "one" (one index per bag) or "uniform" (length U{lmin..lmax})
    lmin: int = 1
    lmax: int = 1
    alpha: Optional[float] = None   # Zipf exponent, None = uniform ids
    weighted: bool = False
    n_bins: int = 200
    n_steps: int = 100

    @property
    def n_tables(self) -> int:
        return len(self.rows)

    @property
    def total_rows(self) -> int:
        return int(sum(self.rows))


def log_uniform_rows(workload: int, n_tables: int, lo: float, hi: float, cap: int,
                     target_total: int) -> tuple:
    """Row counts u_t = exp(U(ln lo, ln hi)), scaled by one common factor c
    (found by bisection) so that sum(clip(round(c * u_t), 3, cap)) meets the
    stated total.  The unscaled draw's expected total falls far short of the
    totals the workloads state, so the scale factor reconciles the two."""
    g = rng(workload, S_ROWCOUNTS)
    u = np.exp(g.uniform(math.log(lo), math.log(hi), size=n_tables))

    def total(c):
        return int(np.clip(np.round(c * u), 3, cap).sum())

    a, b = 1e-6, 1e6
    for _ in range(200):
        m = math.sqrt(a * b)
        if total(m) < target_total:
            a = m
        else:
            b = m
    rows = np.clip(np.round(b * u), 3, cap).astype(np.int64)
    return tuple(int(r) for r in rows)


def _workloads() -> List[Workload]:
    return [
        Workload(1, "tiny: 4 tables x 1000 rows, d=16, INT4 range, batch 128, one-hot uniform ids, sum",
                 rows=(1000,) * 4, dim=16, values=Values("normal", 0.05), bits=(4,), clip="range",
                 batch=128, pooling="one", alpha=None),
        Workload(2, "CTR one-hot: 26 tables log-uniform rows (~34M), d=16, INT4 greedy, batch 2048, "
                    "Zipf 1.05, sum",
                 rows=log_uniform_rows(2, 26, 3, 1e7, 10_000_000, 34_000_000), dim=16,
                 values=Values("normal", 0.02), bits=(4,), clip="greedy", batch=2048, pooling="one",
                 alpha=1.05),
        Workload(3, "large CTR one-hot: 26 tables log-uniform rows (~250M), d=64, 0.1% 10-sigma "
                    "outliers, INT4 range, batch 8192, Zipf 1.1, sum",
                 rows=log_uniform_rows(3, 26, 3, 4e7, 40_000_000, 250_000_000), dim=64,
                 values=Values("outliers", 0.02), bits=(4,), clip="range", batch=8192,
                 pooling="one", alpha=1.1),
        Workload(4, "multi-hot: 64 tables x 1M rows, d=128, INT4/INT8 range, batch 16384, "
                    "bag length U{1..64}, Zipf 1.05, weighted sum",
                 rows=(1_000_000,) * 64, dim=128, values=Values("normal", 0.02), bits=(4, 8),
                 clip="range", batch=16384, pooling="uniform", lmin=1, lmax=64, alpha=1.05,
                 weighted=True),
        Workload(5, "quantizer: one table 5e7 x 64, 99% N(0,0.02) / 1% Laplace(0,0.2), INT4 greedy "
                    "(100 steps) and range, then dequantize",
                 rows=(50_000_000,), dim=64, values=Values("mixture", 0.02), bits=(4,), clip="greedy",
                 batch=0, pooling="one"),
    ]


WORKLOADS = {w.id: w for w in _workloads()}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def scaled(w: Workload, rows: Optional[Sequence[int]] = None, batch: Optional[int] = None) -> Workload:
    """Same workload with fewer rows and/or a smaller batch (oracle-sized cases)."""
    kw = {}
    if rows is not None:
        kw["rows"] = tuple(int(r) for r in rows)
    if batch is not None:
        kw["batch"] = int(batch)
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------------------------
# table values
# ---------------------------------------------------------------------------

def _np_chunk(w: Workload, table: int, chunk: int, n: int) -> np.ndarray:
    v = w.values
    g = rng(w.id, S_VALUES, table, chunk)
    x = g.standard_normal((n, w.dim), dtype=np.float32) * np.float32(v.sigma)
    if v.kind == "outliers":
        hit = g.random((n, w.dim)) < v.p_out
        sign = np.where(g.random((n, w.dim)) < 0.5, -1.0, 1.0)
        x = np.where(hit, (sign * v.out_mult * v.sigma).astype(np.float32), x)
    elif v.kind == "mixture":
        pick = g.random((n, w.dim)) < v.p_mix
        lap = g.laplace(0.0, v.lap_scale, size=(n, w.dim)).astype(np.float32)
        x = np.where(pick, lap, x)
    return np.ascontiguousarray(x, dtype=np.float32)


def table_values_np(w: Workload, table: int, row0: int = 0, nrows: Optional[int] = None) -> np.ndarray:
    """Host (numpy) values of rows [row0, row0+nrows) of one table."""
    n_t = w.rows[table]
    if nrows is None:
        nrows = n_t - row0
    out = np.empty((nrows, w.dim), dtype=np.float32)
    r = row0
    while r < row0 + nrows:
        c = r // CHUNK_ROWS
        c0 = c * CHUNK_ROWS
        cn = min(CHUNK_ROWS, n_t - c0)
        take = min(c0 + cn, row0 + nrows) - r
        blk = _np_chunk(w, table, c, cn)
        out[r - row0:r - row0 + take] = blk[r - c0:r - c0 + take]
        r += take
    return out


def table_values_torch(w: Workload, table: int, row0: int, nrows: int, device: str, out=None):
    """Device values of rows [row0, row0+nrows) of one table, drawn with torch's
    generator on ``device`` in chunks of 2^20 rows (row0 must be chunk-aligned).
    A different generator than the numpy one: values differ from
    table_values_np, so a test uses one or the other for both sides."""
    import torch
    assert row0 % CHUNK_ROWS == 0
    v = w.values
    if out is None:
        out = torch.empty((nrows, w.dim), dtype=torch.float32, device=device)
    g = torch.Generator(device=device)
    r = 0
    while r < nrows:
        c = (row0 + r) // CHUNK_ROWS
        n = min(CHUNK_ROWS, nrows - r)
        g.manual_seed(torch_seed(w.id, S_VALUES, table, c))
        blk = out[r:r + n]
        torch.randn((n, w.dim), generator=g, device=device, out=blk)
        blk.mul_(v.sigma)
        if v.kind == "outliers":
            u = torch.rand((n, w.dim), generator=g, device=device)
            s = torch.rand((n, w.dim), generator=g, device=device)
            val = torch.where(s < 0.5, -v.out_mult * v.sigma, v.out_mult * v.sigma).float()
            torch.where(u < v.p_out, val, blk, out=blk)
            del u, s, val
        elif v.kind == "mixture":
            u = torch.rand((n, w.dim), generator=g, device=device)
            e = torch.rand((n, w.dim), generator=g, device=device, dtype=torch.float64) - 0.5
            e.clamp_(-0.5 + 2.0**-40, 0.5 - 2.0**-40)
            lap = (-v.lap_scale * torch.sign(e) * torch.log1p(-2.0 * e.abs())).float()
            torch.where(u < v.p_mix, lap, blk, out=blk)
            del u, e, lap
        r += n
    return out


# ---------------------------------------------------------------------------
# sparse ids, bag lengths, weights
# ---------------------------------------------------------------------------

_cdf_cache = {}


def _zipf_cdf(n: int, alpha: float) -> np.ndarray:
    key = (n, alpha)
    if key not in _cdf_cache:
        k = np.arange(1, n + 1, dtype=np.float64)
        p = k ** (-alpha)
        c = np.cumsum(p)
        c /= c[-1]
        _cdf_cache.clear()
        _cdf_cache[key] = c
    return _cdf_cache[key]


def scatter_multiplier(n: int) -> int:
    """First integer >= floor(0.618 n) that is coprime to n (1 for n <= 2)."""
    if n <= 2:
        return 1
    a = max(1, int(math.floor(0.618 * n)))
    while math.gcd(a, n) != 1:
        a += 1
    return a


def zipf_ids(n_rows: int, count: int, alpha: Optional[float], g: np.random.Generator) -> np.ndarray:
    """`count` row ids of a table with n_rows rows.  alpha=None: uniform.
    Otherwise rank k in 1..n has probability proportional to k^-alpha (exact
    inverse CDF), and rank k maps to row ((k-1) * a) mod n with a coprime to n,
    so hot rows are scattered through the table as hashed ids would be."""
    if alpha is None:
        return g.integers(0, n_rows, size=count, dtype=np.int64)
    cdf = _zipf_cdf(n_rows, alpha)
    u = g.random(count)
    rank0 = np.searchsorted(cdf, u, side="right")
    rank0 = np.minimum(rank0, n_rows - 1).astype(np.int64)
    a = scatter_multiplier(n_rows)
    return (rank0 * a) % n_rows


@dataclasses.dataclass
class Batch:
    """CSR bags of one batch: bag g = t * B + b covers [offsets[g], offsets[g+1])."""
    indices: np.ndarray        # [nnz] local row ids
    offsets: np.ndarray        # [T*B + 1]
    weights: Optional[np.ndarray]
    table_offsets: np.ndarray  # [T+1] int64 row prefix sums
    B: int
    T: int

    @property
    def nnz(self) -> int:
        return int(self.indices.size)


def batch(w: Workload, batch_seed: int = 0, index_dtype=np.int32, batch_size: Optional[int] = None) -> Batch:
    B = w.batch if batch_size is None else batch_size
    T = w.n_tables
    lengths = []
    ids = []
    for t in range(T):
        if w.pooling == "one":
            L = np.ones(B, dtype=np.int64)
        else:
            L = rng(w.id, S_LENGTHS, t, batch_seed).integers(w.lmin, w.lmax + 1, size=B, dtype=np.int64)
        lengths.append(L)
        ids.append(zipf_ids(w.rows[t], int(L.sum()), w.alpha, rng(w.id, S_INDICES, t, batch_seed)))
    lengths = np.concatenate(lengths)
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    indices = np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)
    weights = None
    if w.weighted:
        weights = np.concatenate([
            rng(w.id, S_WEIGHTS, t, batch_seed).random(int(lengths[t * B:(t + 1) * B].sum()),
                                                        dtype=np.float32)
            for t in range(T)]) if T else np.zeros(0, np.float32)
    table_offsets = np.zeros(T + 1, dtype=np.int64)
    np.cumsum(np.asarray(w.rows, dtype=np.int64), out=table_offsets[1:])
    if index_dtype == np.int32:
        if (indices.size and int(indices.max()) >= 2**31) or int(offsets[-1]) >= 2**31:
            raise ValueError("ids or offsets do not fit int32")
    return Batch(indices.astype(index_dtype), offsets.astype(index_dtype), weights,
                 table_offsets, B, T)
