"""The no-allocation compression entry point (qemb_compress_pooled_noalloc,
through the C ABI) against the entry point that takes a caller workspace
(qemb_compress_pooled): offsets and records identical byte for byte, on two
calls in a row, the second with fewer vectors (the library's fixed array
keeps the first call's contents), and again after a larger call; sizes above
the maximum are refused before any GPU work."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_common import dev, host, require_gpu, special_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    return require_gpu()


def _inputs(g, n, dim, T):
    x = special_rows(g, n, dim)
    x[np.abs(x) > 1e4] = 0.25
    eb = (10.0 ** g.uniform(-4, -1, size=T)).astype(np.float32)
    return dev(x), dev(eb)


def _both(q, x, eb, T):
    import torch
    n, dim = x.shape
    cap = q.compress_bound(n, dim)
    o1 = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda")
    f1 = torch.full((n + 1,), -7, dtype=torch.int64, device="cuda")
    q.compress_pooled(x, eb, T, out=o1, offs=f1)
    o2 = torch.full((cap,), 0x5A, dtype=torch.uint8, device="cuda")
    f2 = torch.full((n + 1,), -9, dtype=torch.int64, device="cuda")
    q.compress_pooled_noalloc(x, eb, o2, f2, T)
    torch.cuda.synchronize()
    a, b = host(f1), host(f2)
    assert np.array_equal(a, b), "offsets differ"
    total = int(a[-1])
    assert np.array_equal(host(o1)[:total], host(o2)[:total]), "records differ"
    return total


@pytest.mark.parametrize("dim", [16, 64, 128, 300])
def test_noalloc_matches_workspace_entry_point(q, dim):
    g = np.random.default_rng(3100 + dim)
    T = 4
    n1, n2 = 64 * 97 + 5, 1000  # the second call smaller than the first
    x1, eb = _inputs(g, n1, dim, T)
    x2, _ = _inputs(g, n2, dim, T)
    assert _both(q, x1, eb, T) > 0
    assert _both(q, x2, eb, T) > 0
    assert _both(q, x1, eb, T) > 0


def test_noalloc_multi_hot_pooled_output_size(q):
    """The multi-hot workload's pooled output (16384 x 64 vectors of d=128),
    then a batch of 1000 x 26 vectors of d=64."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    T = 64
    x = torch.randn((16384, T, 128), generator=g, device="cuda") * 0.05
    eb = torch.full((T,), 1e-3, dtype=torch.float32, device="cuda")
    assert _both(q, x.view(-1, 128), eb, T) > 0
    del x
    x = torch.randn((1000, 26, 64), generator=g, device="cuda") * 0.05
    eb = torch.full((26,), 2e-3, dtype=torch.float32, device="cuda")
    assert _both(q, x.view(-1, 64), eb, 26) > 0


def test_noalloc_empty_and_too_large(q):
    import torch
    x = torch.empty((0, 32), dtype=torch.float32, device="cuda")
    eb = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.empty(16, dtype=torch.uint8, device="cuda")
    offs = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    q.compress_pooled_noalloc(x, eb, out, offs, 1)
    assert int(offs[0].item()) == 0
    lib = q.load_library()
    n = q.COMPRESS_NOALLOC_MAX_VECTORS + 1
    big = torch.empty(16, dtype=torch.float32, device="cuda")
    rc = lib.qemb_compress_pooled_noalloc(big.data_ptr(), n, 32, 1, eb.data_ptr(), out.data_ptr(),
                                          offs.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == -5
    assert int(offs[0].item()) == 0
