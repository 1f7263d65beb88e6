"""GPU parity of the dot interaction of the pooled embeddings ("Deep Learning
Recommendation Model ..." review page, "Proposed method": second-order
interactions are dot products between the embedding vectors and the dense
features, concatenated with the dense features) against the CPU oracle.

Bars: the dense part bit-exact; each dot within
dim * 2^-23 * sum_k |z_ik z_jk| of the oracle's binary64 value -- the
classical bound for a dot product accumulated in binary32 in any order
(dim * 2^-24 per term, Higham's gamma_dim), doubled to leave room for the
matrix cores' internal rounding.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from int4_row_wise_amd import synth
from tests.gpu_common import assert_pooled_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    return require_gpu()


def assert_interaction_close(got, ref, absd, dim, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.array_equal(got[:, :dim].astype(np.float64), ref[:, :dim]), what + ": dense part"
    err = np.abs(got[:, dim:].astype(np.float64) - ref[:, dim:])
    tol = dim * 2.0 ** -23 * absd[:, dim:] + 1e-37
    bad = err > tol
    assert not bad.any(), "%s: %d dots out of tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), float((err / tol).max()))


def _inputs(g, B, T, dim):
    dense = (g.standard_normal((B, dim)) * g.uniform(0.01, 3.0, size=(B, 1))).astype(np.float32)
    pooled = (g.standard_normal((B, T, dim)) * g.uniform(0.001, 10.0, size=(B, T, 1))).astype(np.float32)
    if B > 2 and T > 2:
        pooled[1, 2] = 0.0                    # an all-zero table vector
        pooled[2, :, : max(1, dim // 3)] = -0.0
        dense[0] = 0.0
    return dense, pooled


@pytest.mark.parametrize("T,dim", [(0, 16), (1, 1), (1, 16), (2, 3), (3, 5), (15, 16), (16, 16),
                                   (17, 17), (26, 64), (33, 100), (48, 128), (63, 128), (64, 128),
                                   (64, 127), (64, 4), (65, 128), (40, 129), (100, 64), (26, 256),
                                   (8, 1000), (200, 32), (61, 128), (57, 100), (50, 68),
                                   (49, 72), (4, 1024), (1024, 8)])
def test_interaction_matches_oracle(q, T, dim):
    print("interaction T=%d dim=%d" % (T, dim), flush=True)
    g = np.random.default_rng(9000 + T * 31 + dim)
    B = 37 if T < 512 else 5  # T = 1024: 2 MB of output per sample
    dense, pooled = _inputs(g, B, T, dim)
    ref, absd = oracle.dot_interaction(dense, pooled)
    got = host(q.dot_interaction(dev(dense), dev(pooled)))
    assert_interaction_close(got, ref, absd, dim, "T=%d dim=%d" % (T, dim))


def test_interaction_single_sample_and_empty_batch(q):
    import torch
    g = np.random.default_rng(9100)
    dense, pooled = _inputs(g, 1, 64, 128)
    ref, absd = oracle.dot_interaction(dense, pooled)
    assert_interaction_close(host(q.dot_interaction(dev(dense), dev(pooled))), ref, absd, 128, "B=1")
    e = q.dot_interaction(torch.zeros((0, 128), device="cuda"), torch.zeros((0, 64, 128), device="cuda"))
    assert tuple(e.shape) == (0, q.interaction_width(64, 128))


def test_interaction_deterministic_and_exact_scaling(q):
    """Two runs agree bitwise; scaling dense by 2 doubles exactly the dots
    with the dense vector and leaves the others unchanged."""
    g = np.random.default_rng(9200)
    B, T, dim = 300, 64, 128
    dense, pooled = _inputs(g, B, T, dim)
    d1 = dev(dense)
    p1 = dev(pooled)
    a = host(q.dot_interaction(d1, p1))
    b = host(q.dot_interaction(d1, p1))
    c = host(q.dot_interaction(dev(dense * np.float32(2)), p1))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    i, j = np.tril_indices(T + 1, -1)
    with_dense = np.concatenate([np.zeros(dim, bool), j == 0])
    assert np.array_equal(c[:, with_dense], 2 * a[:, with_dense])
    assert np.array_equal(c[:, ~with_dense & (np.arange(a.shape[1]) >= dim)],
                          a[:, ~with_dense & (np.arange(a.shape[1]) >= dim)])


def test_interaction_multi_hot_shape(q):
    """The multi-hot workload's sample shape (64 tables, d=128) over 2000
    samples whose pooled vectors look like sums of 1..64 weighted rows."""
    g = np.random.default_rng(9300)
    B, T, dim = 2000, 64, 128
    lens = g.integers(1, 65, size=(B, T, 1))
    pooled = (g.standard_normal((B, T, dim)) * 0.02 * np.sqrt(lens / 3.0)).astype(np.float32)
    dense = g.standard_normal((B, dim)).astype(np.float32)
    ref, absd = oracle.dot_interaction(dense, pooled)
    got = host(q.dot_interaction(dev(dense), dev(pooled)))
    assert_interaction_close(got, ref, absd, dim, "multi-hot shape")


def test_lookup_then_interaction(q):
    """The GPU lookup's pooled output fed straight into the interaction,
    against the oracle's lookup and interaction: each dot may differ by the
    propagation of the lookup's tolerance plus the interaction's own bound."""
    import torch
    w = synth.scaled(synth.workload(4), rows=(1000,) * 64, batch=64)
    x = np.concatenate([synth.table_values_np(w, t, 0, w.rows[t]) for t in range(w.n_tables)])
    packed = oracle.quantize_rowwise(x, 4)
    bt = synth.batch(w)
    pooled_gpu = q.bag_forward(dev(packed), dev(bt.table_offsets), bt.B, w.dim, 4, dev(bt.indices),
                               dev(bt.offsets), dev(bt.weights))
    g = np.random.default_rng(9400)
    dense = g.standard_normal((bt.B, w.dim)).astype(np.float32)
    got = host(q.dot_interaction(dev(dense), pooled_gpu))
    pref, pabs, _ = oracle.bag_forward(packed, bt.table_offsets, bt.B, w.dim, 4, bt.indices, bt.offsets,
                                       bt.weights)
    assert_pooled_close(host(pooled_gpu), pref, pabs, "pooled")
    ptol = 1e-5 * pabs + 1e-6                   # the lookup's bound, per element
    pf = pref.astype(np.float32)                 # oracle pooled rounded to the interaction's input
    ptol = ptol + np.abs(pref - pf)
    ref, absd = oracle.dot_interaction(dense, pf)
    Z = np.concatenate([dense[:, None, :].astype(np.float64), pf.astype(np.float64)], axis=1)
    Zt = np.concatenate([np.zeros((bt.B, 1, w.dim)), ptol], axis=1)
    i, j = np.tril_indices(w.n_tables + 1, -1)
    prop = (np.einsum("bpk,bpk->bp", Zt[:, i], np.abs(Z[:, j]) + Zt[:, j]) +
            np.einsum("bpk,bpk->bp", np.abs(Z[:, i]), Zt[:, j]))
    err = np.abs(got[:, w.dim:].astype(np.float64) - ref[:, w.dim:])
    tol = prop + w.dim * 2.0 ** -23 * (absd[:, w.dim:] + prop) + 1e-30
    assert np.all(err <= tol), float((err / tol).max())
    assert np.array_equal(got[:, :w.dim], dense)
