"""HIP graph capture of the library's calls.  The library allocates nothing,
never synchronizes and launches only kernels (no memset or copy nodes), so a
chain of lookup -> compression -> decompression -> dot interaction captured
once replays on new inputs.  Every replay, with new ids, weights and bounds
copied into the captured input tensors and eager work between replays, is
compared bit for bit with the same chain run eagerly on the same inputs
(every kernel of the chain is deterministic)."""
from __future__ import annotations

import numpy as np
import pytest

from int4_row_wise_amd import synth
from tests.gpu_common import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    return require_gpu()


def test_captured_chain_replays(q):
    import torch
    w = synth.scaled(synth.workload(4), rows=(3000,) * 8, batch=256)
    x = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    packed = q.quantize_rowwise(dev(x), 4)
    toff = dev(np.concatenate([[0], np.cumsum(w.rows)]).astype(np.int64))
    B, T, d = w.batch, w.n_tables, w.dim
    batches = [synth.batch(w, batch_seed=k) for k in range(4)]
    cap = max(b.nnz for b in batches)
    g = np.random.default_rng(14000)
    bounds = [(g.uniform(0.2, 2.0, size=T) * 10.0 ** -k).astype(np.float32) for k in (1, 2, 3, 2)]
    dense_np = g.standard_normal((B, d)).astype(np.float32)

    def padded(b):
        idx = np.zeros(cap, np.int32)
        idx[: b.nnz] = b.indices
        wt = np.zeros(cap, np.float32)
        wt[: b.nnz] = b.weights
        return idx, b.offsets.astype(np.int32), wt

    # captured inputs and outputs (fixed addresses)
    idx_s = torch.zeros(cap, dtype=torch.int32, device="cuda")
    off_s = torch.zeros(T * B + 1, dtype=torch.int32, device="cuda")
    wt_s = torch.zeros(cap, dtype=torch.float32, device="cuda")
    eb_s = torch.zeros(T, dtype=torch.float32, device="cuda")
    dense_s = dev(dense_np)
    out_s = torch.empty((B, T, d), dtype=torch.float32, device="cuda")
    n = B * T
    buf_s = torch.empty(q.compress_bound(n, d), dtype=torch.uint8, device="cuda")
    coffs_s = torch.empty(n + 1, dtype=torch.int64, device="cuda")
    ws_s = torch.empty(q.compress_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    y_s = torch.empty((n, d), dtype=torch.float32, device="cuda")
    ix_s = torch.empty((B, q.interaction_width(T, d)), dtype=torch.float32, device="cuda")

    def chain(idx, off, wt, eb, out, buf, coffs, ws, y, ix):
        q.bag_forward(packed, toff, B, d, 4, idx, off, wt, out=out)
        q.compress_pooled(out, eb, out=buf, offs=coffs, workspace=ws)
        q.decompress_pooled(buf, coffs, d, eb, y=y)
        q.dot_interaction(dense_s, out, out=ix)

    def load(k):
        idx, off, wt = padded(batches[k])
        idx_s.copy_(torch.from_numpy(idx))
        off_s.copy_(torch.from_numpy(off))
        wt_s.copy_(torch.from_numpy(wt))
        eb_s.copy_(torch.from_numpy(bounds[k]))

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        chain(idx_s, off_s, wt_s, eb_s, out_s, buf_s, coffs_s, ws_s, y_s, ix_s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(idx_s, off_s, wt_s, eb_s, out_s, buf_s, coffs_s, ws_s, y_s, ix_s)
    torch.cuda.synchronize()

    for rep, k in enumerate([1, 2, 0, 3, 1]):
        print("graph replay %d (batch %d)" % (rep, k), flush=True)
        load(k)
        graph.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in (out_s, coffs_s, y_s, ix_s)]
        got_buf = host(buf_s)[: int(got[1][-1])].copy()
        # eager run of the same chain on fresh buffers, with eager work before it
        idx, off, wt = padded(batches[k])
        e_out = torch.full((B, T, d), 7.0, device="cuda")
        e_buf = torch.zeros_like(buf_s)
        e_coffs = torch.zeros_like(coffs_s)
        e_ws = torch.zeros_like(ws_s)
        e_y = torch.zeros_like(y_s)
        e_ix = torch.zeros_like(ix_s)
        chain(dev(idx), dev(off), dev(wt), dev(bounds[k]), e_out, e_buf, e_coffs, e_ws, e_y, e_ix)
        torch.cuda.synchronize()
        ref = [host(t) for t in (e_out, e_coffs, e_y, e_ix)]
        for a, b, name in zip(got, ref, ("pooled", "offsets", "decompressed", "interaction")):
            assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                  np.ascontiguousarray(b).view(np.uint8)), (rep, name)
        assert np.array_equal(got_buf, host(e_buf)[: int(ref[1][-1])]), (rep, "records")
