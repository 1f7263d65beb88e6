"""Shared helpers of the GPU parity tests (inputs and comparisons only)."""
from __future__ import annotations

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_row_wise_amd import build
    build.ensure_built()
    import int4_row_wise_amd as q
    q.load_library()
    return q


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def special_rows(g: np.random.Generator, rows: int, dim: int) -> np.ndarray:
    """Seeded rows mixing ordinary Gaussian rows with the cases the rules
    single out: constant rows, signed zeros, values below fp16 resolution,
    values near the fp16 limit, two-valued rows, heavy tails."""
    x = (g.standard_normal((rows, dim)) * 0.02).astype(np.float32)
    kinds = g.integers(0, 10, size=rows)
    for r in range(rows):
        k = kinds[r]
        if k == 1:
            x[r] = np.float32(g.standard_normal() * 0.1)
        elif k == 2:
            x[r] = 0.0
            x[r, g.integers(0, dim, size=max(1, dim // 3))] = np.float32(-0.0)
        elif k == 3:
            x[r] *= np.float32(1e-7)
        elif k == 4:
            x[r] = (g.standard_normal(dim) * 20000.0).clip(-65504, 65504).astype(np.float32)
        elif k == 5:
            x[r] = np.where(g.random(dim) < 0.5, -1.5, 2.25).astype(np.float32)
        elif k == 6:
            x[r] = g.laplace(0, 0.2, size=dim).astype(np.float32)
        elif k == 7:
            x[r] = (g.integers(-8, 8, size=dim) * 0.125).astype(np.float32)
        elif k == 8:
            x[r] *= np.float32(300.0)
    return x


def assert_pooled_close(got, ref, absd, what=""):
    """|gpu - oracle| <= 1e-5 * sum|terms| + 1e-6, element by element."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    tol = 1e-5 * absd + 1e-6
    bad = err > tol
    assert not bad.any(), "%s: %d elements out of tolerance, worst excess %.3g (err %.3g)" % (
        what, int(bad.sum()), float((err - tol).max()), float(err.max()))
    return float((err / tol).max()) if err.size else 0.0
